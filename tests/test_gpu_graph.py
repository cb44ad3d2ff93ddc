"""HIP-graph capture of the fixed-shape denoising step.

The serving recipe captures the fixed-shape denoising step in graphs once the prefix
cache exists (vLLM recipe "Qwen/Qwen-Image-2.1", section "CUDA graphs"); here the cache
stays in place and the captured step is one qi_denoise_attn_step per layer on the
caller's stream.  libqi enqueues only kernel launches on that stream (no allocation, no
synchronisation, no memset), so the step captures as it is.  Every replay must reproduce
the eager result bit for bit, with eager work and synchronisation between replays, and a
replay must read the inputs' current contents.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_causal_attention_qi_amd import qi, synth
from oracle import layout as L
from qi_gpu import BF16_MAXABS, BF16_RELRMS, GpuWave, check, exact_inputs, f64, oracle_rows, say

pytestmark = pytest.mark.gpu

WAVES = {
    "ragged": [[40, 70, 96], [23, 129]],    # two requests, ragged blocks, one reference image
    # 1700 keys on 2 heads: the plan cuts the keys into chunks, so the captured step holds
    # the attention kernel and the merge of the chunks
    "chunked": [[100, 700, 900]],
}


def bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("wave", sorted(WAVES))
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_replay_matches_eager(gpu_device, kv, wave):
    layers = [GpuWave(synth.custom(WAVES[wave], 2, 128, kv, seed=300 + l), gpu_device)
              for l in range(3)]
    items = qi.qi_plan_launch_items(layers[0].plan, qi.QI_CALL_DENOISE)
    assert bool((items[:, 4] > 0).any()) == (wave == "chunked")
    for gw in layers:
        gw.build()
    outs = [torch.empty_like(gw.img[0][0]) for gw in layers]

    def step():
        for gw, o in zip(layers, outs):
            q, k, v = gw.img[0]
            qi.qi_denoise_attn_step(gw.plan, gw.cache, q, k, v, o)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(bits(o), bits(r)), ("replay", rep, "layer", l)
        say("  replay %d matches eager (%s cache)" % (rep, kv))
        if rep == 0:
            # the replayed step against the fp64 oracle, every element of every layer (an
            # fp8 cache against the oracle run on the dequantised cache, at the bf16 bar)
            for l, (gw, o) in enumerate(zip(layers, outs)):
                w = gw.w
                rows = [list(range(n)) for n in w.image_lens]
                want = np.concatenate(oracle_rows(w, L.CALL_DENOISE, exact_inputs(gw.x), rows, kv))
                check(f64(o), want, BF16_MAXABS, BF16_RELRMS, "graph replay layer %d vs oracle" % l)

    # new image inputs in the captured buffers: the replay reads them
    q0, k0, v0 = layers[0].img[0]
    q0.copy_(torch.flip(q0, dims=[0]))
    v0.copy_(torch.flip(v0, dims=[0]))
    eager = torch.empty_like(outs[0])
    qi.qi_denoise_attn_step(layers[0].plan, layers[0].cache, q0, k0, v0, eager)
    torch.cuda.synchronize()
    assert not torch.equal(bits(eager), bits(ref[0]))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(eager))
    for o, r in zip(outs[1:], ref[1:]):
        assert torch.equal(bits(o), bits(r))
