"""The allocation-free prefix build (qi_prefix_kv_build_noalloc) against the ordinary one.

Callers that cannot allocate device memory (graph capture, tight serving loops) get a
build whose fp8 absmax partials live in the library's static device array instead of the
workspace.  Two calls in a row through the C ABI, the second with a smaller wave, must give
the cache bytes and prefix outputs of qi_prefix_kv_build bit for bit, and a denoising step
after each must agree too (the array keeps the last call's contents, so the second call
must not depend on them).
"""
from __future__ import annotations

import pytest
import torch

from block_causal_attention_qi_amd import qi, synth
from qi_gpu import GpuWave, nan_like

pytestmark = pytest.mark.gpu

WAVES = [
    ([[300, 700, 200], [150, 129], [64, 64, 64, 33]], 8, 128),   # first call: larger
    ([[100, 50, 64]], 4, 64),                                      # second call: smaller
]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


@pytest.mark.parametrize("kv", ["fp8", "fp8_v", "bf16"])
def test_noalloc_build_matches_ordinary_build(gpu_device, kv):
    runs = []
    for reqs, h, d in WAVES:
        x = synth.custom(reqs, h, d, kv_dtype=kv, seed=900 + h)
        runs.append((GpuWave(x, gpu_device, kv=kv), GpuWave(x, gpu_device, kv=kv)))
    outs, snaps = [], []
    for gw_na, gw in runs:
        # poison every workspace byte the plan's tables do not cover, then upload again
        for w in (gw_na, gw):
            w.ws.fill_(0x7F)
            qi.qi_plan_upload(w.plan, w.ws)
        torch.cuda.synchronize()
        snaps.append((gw_na.ws.clone(), gw.ws.clone()))
    for gw_na, _ in runs:   # two allocation-free calls in a row, larger then smaller
        o = nan_like(tuple(gw_na.q_pre.shape), gpu_device)
        gw_na.cache.fill_(0xA5)
        qi.qi_prefix_kv_build_noalloc(gw_na.plan, gw_na.q_pre, gw_na.k_pre, gw_na.v_pre, o,
                                      gw_na.cache)
        outs.append(o)
    for (gw_na, gw), o_na, (s_na, s) in zip(runs, outs, snaps):
        gw.cache.fill_(0xA5)   # same poison: padding between regions is written by neither
        o = gw.build()
        torch.cuda.synchronize()
        n = gw.plan.cache_bytes
        assert torch.equal(gw_na.cache[:n], gw.cache[:n]), "cache bytes differ"
        assert torch.equal(bits(o_na), bits(o)), "prefix outputs differ"
        # the allocation-free build writes no workspace byte the ordinary build leaves
        # alone (both keep the partial softmax states of split key chunks there, when
        # the plan splits keys); the ordinary fp8 build also keeps its absmax partials
        # there, which the allocation-free one keeps in its static array
        ch_na, ch = gw_na.ws != s_na, gw.ws != s
        assert not torch.any(ch_na & ~ch), "the allocation-free build wrote outside the plan's state"
        assert torch.any(ch & ~ch_na).item() == (kv != "bf16")
        d_na, d = gw_na.denoise(), gw.denoise()
        torch.cuda.synchronize()
        assert torch.equal(bits(d_na), bits(d)), "denoising outputs differ"
