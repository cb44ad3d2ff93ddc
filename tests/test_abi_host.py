"""libqi host side, without a GPU: the library loads, exports every call include/qi.h
declares, and its plan (tile maps, cache offsets, sizes, pair counts, argument checks)
matches the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

qi = pytest.importorskip("block_causal_attention_qi_amd.qi",
                         reason="libqi.so not built (run __graft_entry__.build())")

WAVES = [
    ([[32, 64, 64]], 1, 64),
    ([[256, 4096]], 24, 128),
    ([[256, 4096, 4096, 4096, 4096, 4096]], 24, 128),
    ([[512, 4096, 16384]], 2, 128),
    ([[445, 4096], [349] + [4096] * 5, [293, 4096, 4096, 4096, 4096], [71, 3, 5, 1000]], 3, 128),
    ([[1, 1], [7, 130, 1, 129], [300, 3]], 2, 64),
    ([[5] + [17] * 10 + [33]], 1, 128),
]


def _random_small_head_waves(count=10, seed=77):
    """Seeded ragged waves on 1..3 heads: few (row tile, head) items, so the prefix call,
    the denoising call, both or neither cut their keys into chunks."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        reqs = []
        for _ in range(int(rng.integers(1, 4))):
            refs = [int(v) for v in rng.integers(1, 3001, int(rng.integers(0, 4)))]
            reqs.append([int(rng.integers(1, 601))] + refs + [int(rng.integers(1, 3001))])
        out.append((reqs, int(rng.integers(1, 4)), int(rng.choice([64, 128]))))
    return out


RANDOM_WAVES = _random_small_head_waves()


def _declared():
    with open(os.path.join(ROOT, "include", "qi.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qi_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_call():
    names = _declared()
    assert len(names) >= 13
    lib = ctypes.CDLL(qi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(qi.EXPORTS) == set(names)


@pytest.mark.parametrize("reqs,h,d", WAVES)
def test_tile_maps_match_oracle(reqs, h, d):
    for kv in ("bf16", "fp8", "fp8_v"):
        p = qi.Plan(reqs, h, d, kv)
        for call in (qi.QI_CALL_PREFIX, qi.QI_CALL_DENOISE, qi.QI_CALL_FULL):
            tilings = [qi.qi_plan_kernel_tile(p, call), (64, 64), (128, 128), (256, 64)]
            if sum(map(sum, reqs)) < 3000:
                tilings += [(3, 5), (16, 32), (1, 1)]
            for bm, bn in tilings:
                got = qi.qi_plan_tile_map(p, call, bm, bn)
                want = L.wave_tile_map(reqs, call, bm, bn)
                assert np.array_equal(got, want), (call, bm, bn)


@pytest.mark.parametrize("reqs,h,d", WAVES)
def test_cache_layout_and_pairs_match_oracle(reqs, h, d):
    rng = np.random.default_rng(7)
    for kv_name, kv in (("bf16", L.KV_BF16), ("fp8", L.KV_FP8), ("fp8_v", L.KV_FP8_V)):
        p = qi.Plan(reqs, h, d, kv_name)
        regs, total = L.cache_layout(reqs, h, d, kv)
        assert p.cache_bytes == total
        for r, bl in enumerate(reqs):
            lp = sum(bl[:-1])
            toks = sorted({0, lp - 1, int(rng.integers(0, lp))})
            for which in (0, 1):
                for head in sorted({0, h - 1}):
                    for t in toks:
                        assert qi.qi_plan_cache_offset(p, r, which, head, t) == \
                            L.cache_offset(regs, d, kv, r, which, head, t)
            if kv != L.KV_BF16:
                assert qi.qi_plan_cache_offset(p, r, 2, 0, 0) == regs[r]["s_off"]
        for call in (L.CALL_PREFIX, L.CALL_DENOISE, L.CALL_FULL):
            assert qi.qi_plan_pairs(p, call) == sum(L.useful_pairs(b, call) for b in reqs)
            assert qi.useful_flops(p, call) == L.useful_flops(reqs, call, h, d)
        pre, img, tot = qi.qi_plan_tokens(p)
        assert (pre, img, tot) == (sum(sum(b[:-1]) for b in reqs), sum(b[-1] for b in reqs),
                                   sum(map(sum, reqs)))


def _raw_create(n_req, n_refs, bl, h, d, kv):
    refs = (ctypes.c_int32 * max(1, len(n_refs)))(*n_refs)
    blk = (ctypes.c_int32 * max(1, len(bl)))(*bl)
    desc = qi._WaveDesc(n_req, refs, blk, h, d, kv)
    out = ctypes.c_void_p(123)
    st = qi.lib.qi_plan_create(ctypes.byref(desc), ctypes.byref(out))
    if st == 0:
        qi.lib.qi_plan_destroy(out)
    else:
        assert not out.value   # no plan handed out on error
    return st


def test_plan_create_argument_checks():
    ok = _raw_create(1, [1], [3, 4, 5], 2, 64, 0)
    assert ok == qi.QI_OK
    assert _raw_create(0, [1], [3, 4, 5], 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(65, [0] * 65, [1, 1] * 65, 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(64, [0] * 64, [1, 1] * 64, 2, 64, 0) == qi.QI_OK
    assert _raw_create(1, [11], [1] * 13, 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [10], [1] * 12, 2, 64, 0) == qi.QI_OK
    assert _raw_create(1, [-1], [1, 1], 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [1], [3, 0, 5], 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [0], [0, 5], 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [0], [5, -2], 2, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [1], [3, 4, 5], 0, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [1], [3, 4, 5], 129, 64, 0) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [1], [3, 4, 5], 2, 96, 0) == qi.QI_ERR_UNSUPPORTED
    assert _raw_create(1, [1], [3, 4, 5], 2, 256, 0) == qi.QI_ERR_UNSUPPORTED
    assert _raw_create(1, [1], [3, 4, 5], 2, 64, 2) == qi.QI_OK   # V-only fp8 cache
    assert _raw_create(1, [1], [3, 4, 5], 2, 64, 3) == qi.QI_ERR_INVALID_ARG
    assert _raw_create(1, [0], [1 << 23, 1 << 23], 1, 64, 0) == qi.QI_ERR_INVALID_ARG
    # null descriptor / output
    assert qi.lib.qi_plan_create(None, ctypes.byref(ctypes.c_void_p())) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_create(None, None) == qi.QI_ERR_INVALID_ARG


def test_calls_rejected_before_any_launch():
    """Checks that fire on the host before anything is enqueued (fake, never-touched
    device addresses)."""
    p = qi.Plan([[3, 4, 5]], 2, 64)
    A = ctypes.c_void_p(0x10000)
    mis = ctypes.c_void_p(0x10008)
    big = ctypes.c_size_t(1 << 30)
    h = p.handle
    # workspace never uploaded
    assert qi.lib.qi_prefix_kv_build(h, A, A, A, A, A, big, None) == qi.QI_ERR_STATE
    assert qi.lib.qi_attn_full_reference_step(h, A, A, A, A, None) == qi.QI_ERR_STATE
    assert qi.lib.qi_denoise_attn_step(h, A, big, A, A, A, A, None) == qi.QI_ERR_STATE
    # null or misaligned pointers
    assert qi.lib.qi_prefix_kv_build(h, None, A, A, A, A, big, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_prefix_kv_build(h, A, A, mis, A, A, big, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_denoise_attn_step(h, A, big, A, A, A, None, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_attn_full_reference_step(h, A, A, A, mis, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_attn_full_reference_step(None, A, A, A, A, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_upload(h, None, big, None) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_upload(h, A, ctypes.c_size_t(1), None) == qi.QI_ERR_BUFFER_TOO_SMALL
    # host queries
    n = ctypes.c_size_t()
    assert qi.lib.qi_plan_tile_map(h, 3, 4, 4, None, 0, ctypes.byref(n)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_tile_map(h, 2, 0, 4, None, 0, ctypes.byref(n)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_tile_map(h, 2, 4, 4, None, 0, ctypes.byref(n)) == qi.QI_ERR_BUFFER_TOO_SMALL
    assert n.value == 12
    buf = (ctypes.c_uint8 * 11)()
    assert qi.lib.qi_plan_tile_map(h, 2, 4, 4, buf, 11, None) == qi.QI_ERR_BUFFER_TOO_SMALL
    off = ctypes.c_size_t()
    assert qi.lib.qi_plan_cache_offset(h, 1, 0, 0, 0, ctypes.byref(off)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_cache_offset(h, 0, 0, 2, 0, ctypes.byref(off)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_cache_offset(h, 0, 0, 0, 7, ctypes.byref(off)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_cache_offset(h, 0, 2, 0, 0, ctypes.byref(off)) == qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_sizes(None, None, None) == qi.QI_ERR_INVALID_ARG
    for s in range(6):
        assert qi.qi_status_string(s)
    p.close()
    with pytest.raises(qi.QiError):
        _ = p.handle



@pytest.mark.parametrize("reqs,h,d", WAVES + RANDOM_WAVES)
def test_launch_schedule_covers_every_row_once(reqs, h, d):
    """Every (request, head, row, visible key) of a call is computed by exactly one
    workgroup: items never cross a block and hold at most the kernel's row tile, and the
    key chunks of one item tile its visible keys [0, end of its block) in whole 64-key
    tiles; the full call runs each row in the same item shape and key chunks as the prefix
    or denoising call (the reason reuse is bit-exact); workgroup i runs on XCD i % 8, and
    without key chunks the items of one (request, head) stay on one XCD (these waves are
    small enough that cutting a head's row tiles over XCDs would not shorten the launch;
    see test_xcd_dealing_balances_head_shards)."""
    p = qi.Plan(reqs, h, d)
    den = qi.qi_plan_launch_items(p, qi.QI_CALL_DENOISE)
    split_plan = bool(np.any(den[:, 4] > 0))
    shapes = {}
    for call in (qi.QI_CALL_PREFIX, qi.QI_CALL_DENOISE, qi.QI_CALL_FULL):
        items = qi.qi_plan_launch_items(p, call)
        bm, bn = qi.qi_plan_kernel_tile(p, call)
        assert len(items) % 8 == 0
        pad = items[:, 0] < 0
        assert np.all(items[pad] == -1)
        seen = [np.zeros((sum(bl), h), np.int32) for bl in reqs]
        xcd = {}
        chunks = {}
        for i, e in enumerate(items):
            r, hh, r0, nr, k0, k1 = (int(v) for v in e)
            if r < 0:
                continue
            bl = reqs[r]
            ends = np.cumsum(bl)
            b = int(np.searchsorted(ends, r0, side="right"))
            assert 1 <= nr <= bm and r0 + nr <= ends[b], "item crosses a block"
            if call == qi.QI_CALL_PREFIX:
                assert b < len(bl) - 1
            elif call == qi.QI_CALL_DENOISE:
                assert b == len(bl) - 1
            if not split_plan:
                assert xcd.setdefault((r, hh), i % 8) == i % 8
            chunks.setdefault((r, hh, r0, nr), []).append((k0, k1))
        for (r, hh, r0, nr), ks in chunks.items():
            vis = int(np.cumsum(reqs[r])[np.searchsorted(np.cumsum(reqs[r]), r0, side="right")])
            ks.sort()
            assert ks[0][0] == 0 and ks[-1][1] == vis, (ks, vis)
            for (a0, a1), (b0, _) in zip(ks, ks[1:]):
                assert a1 == b0 and a1 % bn == 0, ks
            assert all(a0 < a1 and a0 % bn == 0 for a0, a1 in ks)
            seen[r][r0:r0 + nr, hh] += 1
            key = (r, hh, r0)
            if call == qi.QI_CALL_FULL:
                assert shapes[key] == (nr, ks)
            else:
                shapes[key] = (nr, ks)
        for r, bl in enumerate(reqs):
            lp = sum(bl[:-1])
            rows = {qi.QI_CALL_PREFIX: slice(0, lp), qi.QI_CALL_DENOISE: slice(lp, sum(bl)),
                    qi.QI_CALL_FULL: slice(0, sum(bl))}[call]
            assert np.all(seen[r][rows] == 1)
            assert np.all(np.delete(seen[r], np.arange(sum(bl))[rows], axis=0) == 0)
    n = ctypes.c_size_t()
    assert qi.lib.qi_plan_launch_items(p.handle, 3, None, 0, ctypes.byref(n)) == \
        qi.QI_ERR_INVALID_ARG
    assert qi.lib.qi_plan_launch_items(p.handle, 1, None, 0, ctypes.byref(n)) == \
        qi.QI_ERR_BUFFER_TOO_SMALL
    assert n.value == qi.QI_LAUNCH_ITEM_FIELDS * len(qi.qi_plan_launch_items(p, 1))


@pytest.mark.parametrize("reqs,h,split,pre_split", [
    ([[256] + [4096] * 5], 3, True, True),     # edit4 on one GPU's head shard (3 of 24 heads)
    ([[512, 4096, 16384]], 3, True, True),     # edit2048, head shard: 54 prefix items
    ([[256] + [4096] * 5], 24, False, False),  # edit4, all 24 heads: 384 items fill the chip
    ([[512, 4096, 16384]], 24, False, False),  # edit2048: 432 prefix items
    ([[256, 4096]], 24, False, False),         # t2i1024: 24 prefix items of 4 key tiles
])
def test_key_split_only_for_underfilled_plans(reqs, h, split, pre_split):
    """Keys are split only in a call with fewer (row tile, head) items than the GPU has
    compute units (the prefix and denoising calls decide each for itself); chunks hold at
    least 8 key tiles (an item's last chunk may be shorter) and a split denoising call
    fills whole rounds of one workgroup per CU closely (at least 90% of the last round);
    the workspace grows by one partial state per (chunk, head) slot."""
    p = qi.Plan(reqs, h, 128)
    pre = qi.qi_plan_launch_items(p, qi.QI_CALL_PREFIX)
    pre = pre[pre[:, 0] >= 0]
    assert bool(np.any(pre[:, 4] > 0)) == pre_split
    if pre_split:
        # every chunk but an item's last holds >= 8 key tiles; the split at least doubles
        # the workgroups of an underfilled call
        for (r, hh, r0), ks in _chunks_of(pre).items():
            assert all(k1 - k0 >= 8 * 64 for k0, k1 in ks[:-1]), ks
        assert len(pre) >= 2 * len(_chunks_of(pre))
    items = qi.qi_plan_launch_items(p, qi.QI_CALL_DENOISE)
    live = items[items[:, 0] >= 0]
    chunked = np.any(live[:, 4] > 0)
    assert chunked == split
    if split:
        last = live[:, 5] == live[:, 5].max()
        assert np.all((live[:, 5] - live[:, 4] >= 8 * 64) | last)
        rounds = -(-len(live) // 256)
        assert len(live) >= 0.9 * 256 * rounds, len(live)
        per_xcd = np.bincount([i % 8 for i, e in enumerate(items) if e[0] >= 0], minlength=8)
        assert per_xcd.max() <= 32 * rounds, per_xcd
        slot_bytes = (256 * 128 + 2 * 256) * 4   # fp32 O of a 256-row tile, then m and l
        assert p.workspace_bytes >= len(live) * slot_bytes


def _xcd_loads(items):
    """Work per XCD (key tiles x 128-row blocks) of a launch schedule (workgroup i on XCD
    i % 8), and the XCDs each (request, head) runs on."""
    load = np.zeros(8)
    where = {}
    for i, (r, hh, _r0, nr, k0, k1) in enumerate(items.tolist()):
        if r < 0:
            continue
        load[i % 8] += ((k1 - k0 + 63) // 64) * ((nr + 127) // 128)
        where.setdefault((r, hh), set()).add(i % 8)
    return load, where


@pytest.mark.parametrize("h", [6, 12, 24])
def test_xcd_dealing_balances_head_shards(h):
    """The 2048x2048 edit on 6 or 12 heads (a 4- or 2-way head split of 24): whole
    (request, head) units cannot balance 8 XCDs (12 equal heads leave four XCDs with twice
    the work), so the plan cuts them into runs of row tiles and every XCD gets the same
    work within 2%; on 24 heads whole units already balance and each (request, head)
    stays on one XCD, sharing its L2."""
    p = qi.Plan([[512, 4096, 16384]], h, 128)
    items = qi.qi_plan_launch_items(p, qi.QI_CALL_DENOISE)
    assert not np.any(items[items[:, 0] >= 0][:, 4] > 0), "no key split at these sizes"
    load, where = _xcd_loads(items)
    assert load.max() <= 1.02 * load.mean(), load
    if h == 24:
        assert all(len(x) == 1 for x in where.values())
    else:
        assert any(len(x) > 1 for x in where.values())


def _chunks_of(items):
    """(request, head, first row) -> sorted key ranges of the item's workgroups."""
    out = {}
    for r, hh, r0, _nr, k0, k1 in items.tolist():
        out.setdefault((r, hh, r0), []).append((k0, k1))
    return {k: sorted(v) for k, v in out.items()}


def test_noalloc_build_rejects_plans_beyond_its_scratch():
    """qi_prefix_kv_build_noalloc refuses, before anything is enqueued, a plan whose fp8
    absmax partials (sum of ceil(L_p / 64) * 2 * H floats) exceed its static array; the
    ordinary build has no such limit (fake, never-touched device addresses)."""
    A = ctypes.c_void_p(0x10000)
    big = ctypes.c_size_t(1 << 40)
    over = qi.Plan([[70000, 1]], 128, 64, "fp8")          # 1094 * 2 * 128 = 280064 floats
    assert 1094 * 2 * 128 > qi.QI_NOALLOC_MAX_PARTIALS
    assert qi.lib.qi_prefix_kv_build_noalloc(over.handle, A, A, A, A, A, big, None) == \
        qi.QI_ERR_BUFFER_TOO_SMALL
    # within the limit the next check (workspace never uploaded) answers instead
    under = qi.Plan([[65000, 1]], 128, 64, "fp8")         # 1016 * 2 * 128 = 260096 floats
    assert 1016 * 2 * 128 <= qi.QI_NOALLOC_MAX_PARTIALS
    assert qi.lib.qi_prefix_kv_build_noalloc(under.handle, A, A, A, A, A, big, None) == \
        qi.QI_ERR_STATE
    assert qi.lib.qi_prefix_kv_build(over.handle, A, A, A, A, A, big, None) == qi.QI_ERR_STATE
    assert qi.lib.qi_prefix_kv_build_noalloc(over.handle, None, A, A, A, A, big, None) == \
        qi.QI_ERR_INVALID_ARG
    # a bf16 cache has no partials
    bf = qi.Plan([[70000, 1]], 128, 64, "bf16")
    assert qi.lib.qi_prefix_kv_build_noalloc(bf.handle, A, A, A, A, A, big, None) == \
        qi.QI_ERR_STATE
