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

