"""GPU parity of the HIP path (called through the C ABI) against the fp64 oracle.

Small waves: every output element is compared.  Full-size workloads (the shapes and the
launch configuration the benchmark times): rows sampled across every row tile and block
are compared one by one, and the exactness invariants hold over the whole output.
Cache bytes (bf16 copies, fp8 codes and scales) must match the oracle bit for bit.
"""
import hashlib

import numpy as np
import pytest
import torch

from block_causal_attention_qi_amd import qi, synth
from oracle import attention as A
from oracle import layout as L

from qi_gpu import (BF16_MAXABS, BF16_RELRMS, FP8_DEQ_MAXABS, FP8_DEQ_RELRMS, FP8_MAXABS,
                    FP8_RELRMS, GpuWave, check, errors, exact_inputs, f64, oracle_rows, say,
                    split, sample_rows)

pytestmark = pytest.mark.gpu


def _cache_matches_oracle(gw, e):
    w = gw.w
    kvn = {"bf16": L.KV_BF16, "fp8": L.KV_FP8, "fp8_v": L.KV_FP8_V}[gw.kv]
    img, defined = L.cache_image(w.requests, w.n_heads, w.head_dim, kvn, e["k_pre"], e["v_pre"])
    got = gw.cache.cpu().numpy()
    assert got.size >= img.size
    bad = np.flatnonzero((got[:img.size] != img) & defined)
    assert bad.size == 0, "cache bytes differ at %d places, first at byte %d" % (bad.size, bad[0])


def _fp8_gates(got, ref_deq, ref_unq, what):
    """fp8 caches: against the oracle on the dequantised cache, the stated fp8 bar and the
    bf16 bar; against the unquantised prefix, no further than the quantisation itself
    moves the oracle (plus the bf16 bar), with both distances reported."""
    check(got, ref_deq, FP8_MAXABS, FP8_RELRMS, what + " vs dequantised, fp8 bar")
    check(got, ref_deq, FP8_DEQ_MAXABS, FP8_DEQ_RELRMS, what + " vs dequantised, bf16 bar")
    ma, rr = errors(got, ref_unq)
    qma, qrr = errors(ref_deq, ref_unq)
    say("  %-40s max-abs %.3e  rel-RMS %.3e  (oracle's own quantisation: %.3e / %.3e)"
        % (what + " vs unquantised", ma, rr, qma, qrr))
    assert rr <= qrr + BF16_RELRMS and ma <= qma + BF16_MAXABS, (what, ma, rr, qma, qrr)


def _full_wave_check(x, dev, kv, steps=1):
    """Every output of build, denoise (each step) and full vs the oracle; cache bytes;
    bf16: denoise image rows bit-identical to the full step's image rows."""
    w = x.workload
    gw = GpuWave(x, dev, steps=steps, kv=kv)
    say("wave %s H=%d D=%d kv=%s" % (w.requests, w.n_heads, w.head_dim, kv))
    o_pre = gw.build()
    o_img = [gw.denoise(s) for s in range(steps)]
    o_all = [gw.full(s) for s in range(steps)]
    torch.cuda.synchronize()
    e0 = exact_inputs(x, 0)
    _cache_matches_oracle(gw, e0)
    ref_pre = np.concatenate([A.prefix_step(bl, *[split(w, e0[t], "pre")[r]
                                                  for t in ("q_pre", "k_pre", "v_pre")])
                              for r, bl in enumerate(w.requests)])
    check(f64(o_pre), ref_pre, BF16_MAXABS, BF16_RELRMS, "prefix build")
    for s in range(steps):
        e = exact_inputs(x, s)
        rows = [list(range(n)) for n in w.image_lens]
        ref_den = np.concatenate(oracle_rows(w, L.CALL_DENOISE, e, rows, kv))
        if kv == "bf16":
            check(f64(o_img[s]), ref_den, BF16_MAXABS, BF16_RELRMS, "denoise step %d" % s)
        else:
            _fp8_gates(f64(o_img[s]), ref_den,
                       np.concatenate(oracle_rows(w, L.CALL_DENOISE, e, rows)),
                       "denoise step %d (%s)" % (s, kv))
        rows = [list(range(n)) for n in w.total_lens]
        ref_all = np.concatenate(oracle_rows(w, L.CALL_FULL, e, rows))
        check(f64(o_all[s]), ref_all, BF16_MAXABS, BF16_RELRMS, "full step %d" % s)
        # reuse == full: on a bf16 cache the image rows agree bit for bit
        full_img = np.concatenate([a[lp:] for a, lp in
                                   zip(split(w, o_all[s].cpu().view(torch.int16).numpy(), "all"),
                                       w.prefix_lens)])
        den_bits = o_img[s].cpu().view(torch.int16).numpy()
        if kv == "bf16":
            assert np.array_equal(full_img, den_bits), "denoise differs from full recompute"
        full_pre = np.concatenate([a[:lp] for a, lp in
                                   zip(split(w, o_all[s].cpu().view(torch.int16).numpy(), "all"),
                                       w.prefix_lens)])
        assert np.array_equal(full_pre, o_pre.cpu().view(torch.int16).numpy()), \
            "prefix rows of the full step differ from the build"
    return gw


def test_tiny_workload(gpu_device):
    x = synth.generate("tiny", steps=3)
    _full_wave_check(x, gpu_device, "bf16", steps=3)


RAGGED = [
    ([[37, 5, 130], [1, 200, 64, 1], [300, 129]], 3),
    ([[1, 1]], 2),
    ([[5] + [17] * 10 + [33]], 2),
    ([[128, 128]], 1),
    ([[64, 64, 64], [127, 129, 257]], 2),
    ([[700, 1500, 900]], 2),
    # one image row tile behind a 4000-token text: 2 items, keys cut into 9 chunks of 8
    # key tiles, more than the merge takes in one batch
    ([[4000, 200]], 2),
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_v"])
@pytest.mark.parametrize("case", range(len(RAGGED)))
def test_ragged_waves(gpu_device, case, kv, d):
    reqs, h = RAGGED[case]
    x = synth.custom(reqs, h, d, kv_dtype=kv, seed=100 + case)
    _full_wave_check(x, gpu_device, kv)


def _random_wave(i):
    """Seeded random wave structure: 1..4 requests, 0..4 references each, ragged block
    lengths (text 1..400, references 1..700, image 1..900 tokens), 1..3 heads."""
    rng = np.random.default_rng(1000 + i)
    reqs = []
    for _ in range(int(rng.integers(1, 5))):
        n_refs = int(rng.integers(0, 5))
        reqs.append([int(rng.integers(1, 401))] + [int(v) for v in rng.integers(1, 701, n_refs)]
                    + [int(rng.integers(1, 901))])
    return reqs, int(rng.integers(1, 4))


@pytest.mark.parametrize("i", range(12))
def test_random_waves(gpu_device, i):
    reqs, h = _random_wave(i)
    kv = ("bf16", "fp8", "fp8_v")[i % 3]
    d = (128, 64)[(i // 3) % 2]
    print("random wave %d: %s heads %d d %d kv %s" % (i, reqs, h, d, kv), flush=True)
    x = synth.custom(reqs, h, d, kv_dtype=kv, seed=2000 + i)
    _full_wave_check(x, gpu_device, kv)


def _max_wave(seed):
    """QI_MAX_REQUESTS requests with 0..QI_MAX_REFS references each (every count present)
    and short ragged blocks (1..40 tokens)."""
    rng = np.random.default_rng(seed)
    reqs = []
    for r in range(qi.QI_MAX_REQUESTS):
        n_refs = r % (qi.QI_MAX_REFS + 1)
        reqs.append([int(x) for x in rng.integers(1, 41, size=n_refs + 2)])
    return reqs


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_maximum_wave(gpu_device, kv):
    x = synth.custom(_max_wave(77), 2, 128, kv_dtype=kv, seed=77)
    assert len(x.workload.requests) == qi.QI_MAX_REQUESTS
    _full_wave_check(x, gpu_device, kv)


@pytest.mark.parametrize("d", [64, 128])
def test_maximum_heads(gpu_device, d):
    x = synth.custom([[20, 33, 47], [3, 200]], qi.QI_MAX_HEADS, d, seed=78)
    _full_wave_check(x, gpu_device, "bf16")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_true_cfg_pair(gpu_device, kv):
    """True CFG: the negative-prompt branch runs as a second request of the wave, with its
    own text, the same reference and the same image Q/K/V (vLLM recipe "Qwen/Qwen-Image-2.1",
    section "Sampling defaults": a negative prompt runs the DiT twice per step).  Both
    branches match the oracle; the negative prompt changes the image rows."""
    x = synth.custom([[150, 300, 400]], 3, 128, kv_dtype=kv, seed=41)
    y = synth.cfg_pair(x, 40, seed=42)
    gw = _full_wave_check(y, gpu_device, kv)
    o = gw.denoise()
    torch.cuda.synchronize()
    pos, neg = split(y.workload, f64(o), "img")
    assert pos.shape == neg.shape and not np.array_equal(pos, neg)


# ------------------------------------------------------------------ full-size workloads

@pytest.fixture(scope="module")
def big():
    cache = {}

    def get(name):
        """A named workload, or "<name>@h3": its head shard of three heads."""
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            say("generating %s" % name)
            base, _, shard = name.partition("@h")
            w = synth.head_shard(base, int(shard)) if shard else base
            cache[name] = synth.generate(w, steps=1)
        return cache[name]
    return get


def _sampled(gw, e, call, out, kv, n_random, seed, bar):
    w = gw.w
    rng = np.random.default_rng(seed)
    bm, _ = qi.qi_plan_kernel_tile(gw.plan, call)
    heads = sorted({0, w.n_heads - 1} | set(int(h) for h in rng.integers(0, w.n_heads, 4)))
    items = qi.qi_plan_launch_items(gw.plan, call)
    rows = [sample_rows(bl, call, bm, rng, n_random, items, r) for r, bl in enumerate(w.requests)]
    ref = oracle_rows(w, call, e, rows, kv, heads)
    which = {L.CALL_PREFIX: "pre", L.CALL_DENOISE: "img", L.CALL_FULL: "all"}[call]
    got = [part[np.asarray(r)][:, heads] for part, r in zip(split(w, f64(out), which), rows)]
    name = {0: "prefix", 1: "denoise", 2: "full"}[call]
    what = "%s sampled (%d rows x %d heads)" % (name, sum(map(len, rows)), len(heads))
    if call == L.CALL_DENOISE and kv != "bf16":
        ref_unq = oracle_rows(w, call, e, rows, "bf16", heads)
        return _fp8_gates(np.concatenate(got), np.concatenate(ref), np.concatenate(ref_unq),
                          what + " " + kv)
    return check(np.concatenate(got), np.concatenate(ref), *bar, what)


def _full_size_bf16_check(gw, x):
    """Sampled rows of build, denoise and full vs the oracle; denoise deterministic and
    bit-identical to the full step's image rows; prefix rows of the full step equal to
    the build; the bf16 cache a head-major copy of the prefix K/V."""
    o_pre = gw.build()
    o_img = gw.denoise()
    o_img2 = gw.denoise()
    o_all = gw.full()
    torch.cuda.synchronize()
    e = exact_inputs(x)
    bar = (BF16_MAXABS, BF16_RELRMS)
    _sampled(gw, e, L.CALL_DENOISE, o_img, "bf16", 48, 1, bar)
    _sampled(gw, e, L.CALL_PREFIX, o_pre, "bf16", 24, 2, bar)
    _sampled(gw, e, L.CALL_FULL, o_all, "bf16", 24, 3, bar)
    w = gw.w
    assert torch.equal(o_img.view(torch.int16), o_img2.view(torch.int16)), "not deterministic"
    lp = w.prefix_lens[0]
    assert torch.equal(o_all[lp:].view(torch.int16), o_img.view(torch.int16)), \
        "denoise differs from full recompute"
    assert torch.equal(o_all[:lp].view(torch.int16), o_pre.view(torch.int16))
    # cache bytes: compare the head-major copy with the packed prefix directly on device
    h, d = w.n_heads, w.head_dim
    kc = gw.cache[:h * lp * d * 2].view(torch.bfloat16).view(h, lp, d)
    assert torch.equal(kc.view(torch.int16), gw.k_pre.transpose(0, 1).contiguous().view(torch.int16))
    voff = qi.qi_plan_cache_offset(gw.plan, 0, 1, 0, 0)
    vc = gw.cache[voff:voff + h * lp * d * 2].view(torch.bfloat16).view(h, lp, d)
    assert torch.equal(vc.view(torch.int16), gw.v_pre.transpose(0, 1).contiguous().view(torch.int16))


@pytest.mark.parametrize("name", ["t2i1024", "edit4", "edit2048"])
def test_full_size_bf16(gpu_device, big, name):
    x = big(name)
    gw = GpuWave(x, gpu_device)
    say("%s: requests %s" % (name, gw.w.requests))
    _full_size_bf16_check(gw, x)


def _chunk_items(gw, call):
    items = qi.qi_plan_launch_items(gw.plan, call)
    live = items[items[:, 0] >= 0]
    return live, int(np.sum(live[:, 4] > 0))


@pytest.mark.parametrize("name", ["edit4", "edit2048"])
def test_head_shard_bf16(gpu_device, big, name):
    """One GPU's head shard (3 of 24 heads) at full length: too few (row tile, head)
    items for the chip, so the plan cuts keys into chunks and merges them; the sampled
    rows match the oracle and reuse stays bit-exact through the split."""
    x = big(name + "@h3")
    gw = GpuWave(x, gpu_device)
    live, chunked = _chunk_items(gw, qi.QI_CALL_DENOISE)
    say("%s@h3: %d denoising workgroups, %d of them later key chunks" % (name, len(live), chunked))
    assert chunked > 0, "the head shard did not split keys"
    _full_size_bf16_check(gw, x)


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_head_shard_wave8_request(gpu_device, kv):
    """The wave8 request with the most references, alone, on a three-head shard: key
    chunks over an fp8 (or bf16) cache, sampled rows against the oracle."""
    refs = [len(b) - 2 for b in synth.WORKLOADS["wave8"].requests]
    r = int(np.argmax(refs))
    w = synth.head_shard("wave8", 3, requests=[r])
    x = synth.generate(w, steps=1)
    gw = GpuWave(x, gpu_device, kv=kv)
    live, chunked = _chunk_items(gw, qi.QI_CALL_DENOISE)
    assert chunked > 0
    o_pre = gw.build()
    o_img = gw.denoise()
    o_img2 = gw.denoise()
    torch.cuda.synchronize()
    e = exact_inputs(x)
    _sampled(gw, e, L.CALL_DENOISE, o_img, kv, 24, 8, (BF16_MAXABS, BF16_RELRMS))
    _sampled(gw, e, L.CALL_PREFIX, o_pre, "bf16", 12, 9, (BF16_MAXABS, BF16_RELRMS))
    assert torch.equal(o_img.view(torch.int16), o_img2.view(torch.int16)), "not deterministic"


def test_full_size_wave8_fp8(gpu_device, big):
    x = big("wave8")
    w = x.workload
    gw = GpuWave(x, gpu_device)
    o_pre = gw.build()
    o_img = gw.denoise()
    o_img2 = gw.denoise()
    torch.cuda.synchronize()
    e = exact_inputs(x)
    _sampled(gw, e, L.CALL_DENOISE, o_img, "fp8", 12, 4, None)
    _sampled(gw, e, L.CALL_PREFIX, o_pre, "bf16", 8, 5, (BF16_MAXABS, BF16_RELRMS))
    assert torch.equal(o_img.view(torch.int16), o_img2.view(torch.int16)), "not deterministic"
    # fp8 codes and scales, bit for bit, for one head of every request and all scales
    from oracle import fp8 as F
    cache = gw.cache.cpu().numpy()
    h = w.n_heads
    ks, vs = split(w, e["k_pre"], "pre"), split(w, e["v_pre"], "pre")
    for r in range(len(w.requests)):
        lp = w.prefix_lens[r]
        s_off = qi.qi_plan_cache_offset(gw.plan, r, 2, 0, 0)
        got_sc = cache[s_off:s_off + 8 * h].view("<f4").reshape(2, h)
        for kvi, src in ((0, ks[r]), (1, vs[r])):
            for hh in range(h):
                assert got_sc[kvi, hh] == F.absmax_scale(src[:, hh])[0], (r, kvi, hh)
            hh = r % h
            codes, scale = F.quantize_slab(src[:, hh])
            off = qi.qi_plan_cache_offset(gw.plan, r, kvi, hh, 0)
            got = cache[off:off + lp * w.head_dim].reshape(lp, w.head_dim)
            assert np.array_equal(got, codes), (r, kvi, hh)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp8_v"])
def test_full_size_ten_references(gpu_device, big, kv):
    """The model's maximum of ten references (41,216 prefix tokens) with each cache type;
    bf16 also runs the full recompute and checks that reuse is exact."""
    x = big("edit10")
    w = x.workload
    gw = GpuWave(x, gpu_device, kv=kv)
    o_pre = gw.build()
    o_img = gw.denoise()
    torch.cuda.synchronize()
    e = exact_inputs(x)
    bar = (BF16_MAXABS, BF16_RELRMS)
    _sampled(gw, e, L.CALL_DENOISE, o_img, kv, 24, 6, bar)
    if kv == "bf16":
        _sampled(gw, e, L.CALL_PREFIX, o_pre, "bf16", 24, 7, bar)
        o_all = gw.full()
        torch.cuda.synchronize()
        lp = w.prefix_lens[0]
        assert torch.equal(o_all[lp:].view(torch.int16), o_img.view(torch.int16)), \
            "denoise differs from full recompute"
    else:
        # cache bytes of one head, K and V, against the oracle's encoder
        from oracle import fp8 as F
        cache = gw.cache.cpu().numpy()
        lp, hh, d = w.prefix_lens[0], 5, w.head_dim
        k0, v0 = e["k_pre"][:, hh], e["v_pre"][:, hh]
        vcodes, _ = F.quantize_slab(v0)
        off = qi.qi_plan_cache_offset(gw.plan, 0, 1, hh, 0)
        assert np.array_equal(cache[off:off + lp * d].reshape(lp, d), vcodes)
        off = qi.qi_plan_cache_offset(gw.plan, 0, 0, hh, 0)
        if kv == "fp8":
            kcodes, _ = F.quantize_slab(k0)
            assert np.array_equal(cache[off:off + lp * d].reshape(lp, d), kcodes)
        else:
            kb = cache[off:off + lp * d * 2].view("<u2").reshape(lp, d)
            assert np.array_equal(kb, L.bf16_bits(k0))


# ------------------------------------------------------------------ invariants

def _hash(t):
    return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()


def test_prefix_independence_and_cache_stability(gpu_device):
    x = synth.custom([[100, 300, 300, 250]], 4, 128, seed=7, steps=3)
    gw = GpuWave(x, gpu_device, steps=3)
    o_pre = gw.build()
    torch.cuda.synchronize()
    h0 = _hash(gw.cache)
    outs = [gw.denoise(s) for s in range(3)]
    torch.cuda.synchronize()
    assert _hash(gw.cache) == h0, "a denoising step changed the cache"
    assert not torch.equal(outs[0], outs[1])
    # full step with two different image blocks: prefix rows bit-identical
    a, b = gw.full(0), gw.full(1)
    torch.cuda.synchronize()
    lp = x.workload.prefix_lens[0]
    assert torch.equal(a[:lp].view(torch.int16), b[:lp].view(torch.int16))
    assert torch.equal(a[:lp].view(torch.int16), o_pre.view(torch.int16))
    assert not torch.equal(a[lp:], b[lp:])


def test_request_isolation(gpu_device):
    reqs = [[120, 200, 300], [77, 333], [50, 64, 64, 129]]
    x1 = synth.custom(reqs, 3, 128, seed=8)
    x2 = synth.custom(reqs, 3, 128, seed=8)
    w = x1.workload
    # perturb request 1 everywhere (prefix and image)
    for arr, which in ((x2.q_pre, "pre"), (x2.k_pre, "pre"), (x2.v_pre, "pre"),
                       (x2.q_img[0], "img"), (x2.k_img[0], "img"), (x2.v_img[0], "img")):
        lens = w.prefix_lens if which == "pre" else w.image_lens
        o0 = lens[0]
        arr[o0:o0 + lens[1]] = -arr[o0:o0 + lens[1]] * 1.5
    outs = []
    for x in (x1, x2):
        for kv in ("bf16", "fp8", "fp8_v"):
            gw = GpuWave(x, gpu_device, kv=kv)
            p = gw.build()
            d = gw.denoise()
            f = gw.full()
            torch.cuda.synchronize()
            outs.append((kv, [split(w, t.cpu().view(torch.int16).numpy(), k)
                              for t, k in ((p, "pre"), (d, "img"), (f, "all"))]))
    for i in range(3):
        (_, a), (_, b) = outs[i], outs[i + 3]
        for call in range(3):
            assert np.array_equal(a[call][0], b[call][0]) and np.array_equal(a[call][2], b[call][2])
            assert not np.array_equal(a[call][1], b[call][1])


# ------------------------------------------------------------------ closed forms on device

def test_closed_forms_on_gpu(gpu_device):
    reqs = [[40, 100, 70], [33, 200]]
    x = synth.custom(reqs, 2, 128, seed=9)
    w = x.workload
    # V == 1 everywhere: every output is 1
    ones = synth.WaveInputs(w, x.q_pre, x.k_pre, np.ones_like(x.v_pre), [x.q_img[0]],
                            [x.k_img[0]], [np.ones_like(x.v_img[0])])
    gw = GpuWave(ones, gpu_device)
    outs = [gw.build(), gw.denoise(), gw.full()]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.max(torch.abs(o.float() - 1.0)).item() <= 2.0 ** -8
    # constant K per head: output = mean of the allowed V rows
    kc = np.broadcast_to(x.k_pre[:1], x.k_pre.shape).copy()
    kci = np.broadcast_to(x.k_pre[:1], x.k_img[0].shape).copy()
    const = synth.WaveInputs(w, x.q_pre, kc, x.v_pre, [x.q_img[0]], [kci], [x.v_img[0]])
    gw = GpuWave(const, gpu_device)
    o = gw.full()
    torch.cuda.synchronize()
    v_all = synth.bf16_exact(const.full(0)[2])
    ref = []
    for bl, v in zip(w.requests, split(w, v_all, "all")):
        ends = np.cumsum(bl)
        for p in range(sum(bl)):
            e = int(ends[np.searchsorted(ends, p, side="right")])
            ref.append(v[:e].mean(axis=0))
    check(f64(o), np.stack(ref), BF16_MAXABS, BF16_RELRMS, "constant K -> mean of V")


@pytest.mark.parametrize("kv", ["fp8", "fp8_v"])
def test_fp8_zero_head(gpu_device, kv):
    """A head whose prefix K and V are all zero has absmax 0: its scales are 1 and its
    codes 0 (the quantiser's a == 0 case), and the denoising step still matches the oracle
    on every row; a head with tiny values keeps its relative precision."""
    reqs = [[64, 150, 200], [40, 128]]
    x = synth.custom(reqs, 3, 128, kv_dtype=kv, seed=12)
    x.k_pre[:, 1] = 0.0
    x.v_pre[:, 1] = 0.0
    x.v_pre[:, 2] *= 1e-6
    _full_wave_check(x, gpu_device, kv)
    gw = GpuWave(x, gpu_device, kv=kv)
    gw.build()
    torch.cuda.synchronize()
    cache = gw.cache.cpu().numpy()
    for r in range(len(reqs)):
        s_off = qi.qi_plan_cache_offset(gw.plan, r, 2, 0, 0)
        sc = cache[s_off:s_off + 8 * 3].view("<f4").reshape(2, 3)
        assert sc[0, 1] == 1.0 and sc[1, 1] == 1.0
        off = qi.qi_plan_cache_offset(gw.plan, r, 1, 1, 0)
        assert not cache[off:off + w_lp(reqs[r]) * 128].any()


def w_lp(bl):
    return int(sum(bl[:-1]))


# ------------------------------------------------------------------ errors on device

def test_error_paths_leave_outputs_untouched(gpu_device):
    x = synth.custom([[20, 30, 40]], 2, 64, seed=10)
    gw = GpuWave(x, gpu_device)
    q, k, v = gw.img[0]
    o = torch.full(tuple(q.shape), 7.0, dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(qi.QiError) as ei:                 # denoise before any build
        qi.qi_denoise_attn_step(gw.plan, gw.cache, q, k, v, o)
    assert ei.value.status == qi.QI_ERR_STATE
    small = gw.cache[:gw.plan.cache_bytes - 256]
    op = torch.full(tuple(gw.q_pre.shape), 7.0, dtype=torch.bfloat16, device=gpu_device)
    with pytest.raises(qi.QiError) as ei:
        qi.qi_prefix_kv_build(gw.plan, gw.q_pre, gw.k_pre, gw.v_pre, op, small)
    assert ei.value.status == qi.QI_ERR_BUFFER_TOO_SMALL
    gw.build()
    with pytest.raises(qi.QiError) as ei:
        qi.qi_denoise_attn_step(gw.plan, small, q, k, v, o)
    assert ei.value.status == qi.QI_ERR_BUFFER_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(o == 7.0) and torch.all(op == 7.0)
    qi.qi_denoise_attn_step(gw.plan, gw.cache, q, k, v, o)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
