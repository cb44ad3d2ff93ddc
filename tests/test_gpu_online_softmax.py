"""GPU parity where the online softmax must raise its running maximum late in the key loop.

The kernel computes softmax over the keys one key tile at a time with a running row
maximum m; it raises m (rescaling the partial output and row sum by 2^(m_old - m_new),
strictly between 0 and 1) only when a tile's maximum exceeds m by more than 8 log2 units.
With ordinary unit-RMS rows no later tile ever does, so that correction would only ever
run on the first tile (where the old state is empty).  These waves force it: Q is scaled
by 3 (scores spread over tens of log2 units) and, for chosen image rows, a key is planted
late in the sequence whose score exceeds every earlier score of that row by 10 to 13.5
log2 units (V is scaled by 1/4: a row dominated by one key outputs about that key's V
row, and the absolute bar is stated for outputs below 1).  The planted keys sit in every kind of key tile the denoising step reads: a
tile wholly in the prefix cache (bf16 rows, or E4M3FN codes with folded scales), the tile
that mixes cached and live keys, live image tiles, and the short last tile (masked tail).

The wave has 2304 image rows and 32 heads, so the launch schedule runs some row tiles
whole and splits others in two halves that run with the key tiles split over two groups
of wavefronts (each with its own running maximum, merged at the end); the test checks,
from the schedule the plan reports, that planted rows fall in both kinds of item.  Every
output element of the denoising step is compared with the fp64 oracle (vLLM recipe
"Qwen/Qwen-Image-2.1", section "Prefix KV cache": reuse is exact, so the cached step must
give the softmax of the full sequence).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_causal_attention_qi_amd import qi, synth
from oracle import attention as A
from oracle import layout as L

from qi_gpu import (BF16_MAXABS, BF16_RELRMS, GpuWave, check, errors, exact_inputs, f64,
                    oracle_prefix_values, oracle_rows, say, split)

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634
BLOCKS = [240, 700, 2304]     # text, one reference, image: L_p = 940, N = 3244
HEADS = 32
TAU = 8.0                     # the kernel's raise threshold, log2 units


def _key_kinds(lp, n, bn):
    """Key positions grouped by the kind of key tile holding them (denoising step)."""
    t_mixed = lp // bn
    kinds = {
        "cached": np.arange(2 * bn, t_mixed * bn),                 # tiles wholly cached
        "mixed": np.arange(t_mixed * bn, min(n, (t_mixed + 1) * bn)),
        "live": np.arange((t_mixed + 1) * bn, (n // bn) * bn),
        "partial": np.arange((n // bn) * bn, n),
    }
    assert lp % bn and n % bn and all(v.size for v in kinds.values())
    return kinds


def spiky_wave(d, kv, seed):
    """One request BLOCKS with planted late-key spikes; returns (inputs, plants) where
    plants is a list of (image row, key position, kind)."""
    x = synth.custom([BLOCKS], HEADS, d, kv_dtype=kv, seed=seed)
    x.q_pre *= 3.0
    x.q_img[0] *= 3.0
    # a row dominated by one key outputs about that key's V row, so V is scaled by 1/4 to
    # keep |O| below 1, the range of the workloads' outputs for which the absolute bar is
    # stated (the relative-RMS bar does not depend on the scale)
    x.v_pre *= 0.25
    x.v_img[0] *= 0.25
    bl = BLOCKS
    lp, n = sum(bl[:-1]), sum(bl)
    _, bn = qi.qi_plan_kernel_tile(qi.Plan([bl], HEADS, d, kv), qi.QI_CALL_DENOISE)
    kinds = _key_kinds(lp, n, bn)
    rng = np.random.default_rng(seed + 1)
    names = list(kinds)
    rows = np.arange(0, bl[-1], 23)                       # about 100 planted rows
    used = set()
    plants = []
    for i, row in enumerate(rows):
        for j in range(len(names)):                        # kinds in turn, while keys last
            kind = names[(i + j) % len(names)]
            cand = [int(k) for k in kinds[kind] if int(k) not in used]
            if cand:
                break
        key = int(rng.choice(cand))
        used.add(key)
        plants.append((int(row), key, kind))
    plants.sort(key=lambda p: p[1])                        # earlier keys first
    k_all = np.concatenate([x.k_pre, x.k_img[0]], 0)       # float32 [N, H, D]
    scale = LOG2E / np.sqrt(d)
    for row, key, _ in plants:
        q = x.q_img[0][row].astype(np.float64)             # [H, D]
        t0 = key // bn * bn
        run = np.einsum("hd,khd->hk", q, k_all[:t0].astype(np.float64)).max(axis=1) * scale
        target = run + rng.uniform(10.0, 13.5, HEADS)       # log2 units
        k_all[key] = (q * (target / scale / np.sum(q * q, axis=1))[:, None]).astype(np.float32)
    x.k_pre[:] = k_all[:lp]
    x.k_img[0][:] = k_all[lp:]
    return x, plants, bn


def _exceedance(x, kv, plants, bn):
    """For each planted (row, key): the planted tile's max score of that row minus the
    row's max over every earlier key, log2 units, from the values the kernel reads
    (bf16 inputs; the dequantised cache for fp8), per head.  [n_plants, H]"""
    w = x.workload
    e = exact_inputs(x)
    kp, _ = oracle_prefix_values(w, e, kv)
    k = np.concatenate([kp[0], e["k_img"]], 0)
    scale = LOG2E / np.sqrt(w.head_dim)
    out = []
    for row, key, _ in plants:
        s = np.einsum("hd,khd->hk", e["q_img"][row], k) * scale
        t0 = key // bn * bn
        out.append(s[:, t0:t0 + bn].max(axis=1) - s[:, :t0].max(axis=1))
    return np.asarray(out)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_v"])
def test_late_max_raise(gpu_device, kv, d):
    x, plants, bn = spiky_wave(d, kv, seed=500 + d + {"bf16": 0, "fp8": 1, "fp8_v": 2}[kv])
    w = x.workload
    lp = w.prefix_lens[0]
    exc = _exceedance(x, kv, plants, bn)
    kinds = np.array([p[2] for p in plants])
    for kind in ("cached", "mixed", "live", "partial"):
        # every planted (row, head) of this kind forces a raise with 0 < alpha < 2^-8
        assert np.all(exc[kinds == kind] > TAU + 0.5), (kind, exc[kinds == kind].min())
        assert np.all(exc[kinds == kind] < 60.0)
    gw = GpuWave(x, gpu_device)
    items = qi.qi_plan_launch_items(gw.plan, qi.QI_CALL_DENOISE)
    bm, _ = qi.qi_plan_kernel_tile(gw.plan, qi.QI_CALL_DENOISE)
    item_rows = np.zeros((w.image_lens[0], HEADS), np.int32)   # row count of each row's item
    for r, h, r0, nr in items[items[:, 0] >= 0][:, :4]:
        item_rows[r0 - lp:r0 - lp + nr, h] = nr
    prow = np.array([p[0] for p in plants])
    assert np.any(item_rows[prow] > bm // 2), "no planted row in a whole row tile"
    assert np.any(item_rows[prow] <= bm // 2), "no planted row in a split half"
    say("late max raise kv=%s D=%d: %d planted rows, exceedance %.1f..%.1f log2 units, "
        "%d / %d planted (row, head) in whole tiles" % (
            kv, d, len(plants), exc.min(), exc.max(), int(np.sum(item_rows[prow] > bm // 2)),
            item_rows[prow].size))

    o_pre = gw.build()
    o_img = gw.denoise()
    o_all = gw.full()
    torch.cuda.synchronize()
    e = exact_inputs(x)
    got = f64(o_img)
    ref = oracle_rows(w, L.CALL_DENOISE, e, [list(range(w.image_lens[0]))], kv)[0]
    # every element, at the bf16 bar (fp8: against the dequantised cache the kernel reads)
    check(got, ref, BF16_MAXABS, BF16_RELRMS, "denoise, every element")
    rest = np.setdiff1d(np.arange(w.image_lens[0]), prow)
    check(got[rest], ref[rest], BF16_MAXABS, BF16_RELRMS, "denoise, rows without a spike")
    # planted rows one by one: the spike dominates, the rows keep their own norm
    per_row = np.linalg.norm(got[prow] - ref[prow], axis=2) / np.linalg.norm(ref[prow], axis=2)
    say("  planted rows: worst per-(row, head) relative error %.3e" % per_row.max())
    assert per_row.max() <= 1e-2
    ref_pre = A.prefix_step(BLOCKS, e["q_pre"], e["k_pre"], e["v_pre"])
    check(f64(o_pre), ref_pre, BF16_MAXABS, BF16_RELRMS, "prefix build")
    if kv == "bf16":
        # the full recompute runs the same rows over the same key tiles: bit-identical
        assert torch.equal(o_all[lp:].view(torch.int16), o_img.view(torch.int16))
    else:
        ma, rr = errors(got, oracle_rows(w, L.CALL_DENOISE, e, [list(range(w.image_lens[0]))])[0])
        say("  %-40s max-abs %.3e  rel-RMS %.3e" % ("(vs unquantised prefix, reported)", ma, rr))
    full_img = f64(o_all[lp:])
    ref_full = oracle_rows(w, L.CALL_FULL, e, [list(range(lp, sum(BLOCKS)))])[0]
    check(full_img, ref_full, BF16_MAXABS, BF16_RELRMS, "full step, image rows")
