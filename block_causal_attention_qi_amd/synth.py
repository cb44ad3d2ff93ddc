"""Seeded synthetic inputs for prefix-reuse block-causal attention.

This module holds no part of the attention arithmetic: it only draws inputs.  Both the
HIP path and the fp64 oracle consume what it returns (the oracle through exact float64
widening of the bf16-rounded values), so neither side's results feed the other.

Workloads (block lengths in tokens, order text, ref_1..ref_R, image):
  tiny      1 head x 64, blocks 32 / 64 / 64, 3 denoising steps, seed 0
  t2i1024   24 heads x 128, blocks 256 / 4096 (64x64 latent of a 1024^2 image), seed 1
  edit4     24 x 128, blocks 256 / 4 x 4096 / 4096 (four ~1024^2 references), seed 2
  edit2048  24 x 128, blocks 512 / 4096 / 16384 (128x128 latent of 2048^2), seed 3
  wave8     24 x 128, eight 1024^2 requests at one denoising phase, fp8 prefix cache,
            text lengths and reference counts fixed below, seed 4
Image token count is (height/16) * (width/16): the autoencoder compresses 16x spatially
([recipe] "Overview") and no further patching is assumed.

Row recipe (stands for post-norm DiT activations): x ~ N(0, 1) per element, each
(token, head) row divided by its root-mean-square, then multiplied by a per-(tensor,
head, channel) gain gamma ~ U(0.8, 1.2).  Draw order: gamma for Q, K, V (each [H, D]);
then for every request in wave order the prefix rows of Q, K, V; then for every
denoising step and every request the image rows of Q, K, V.  Values are drawn in
float32 and rounded to bf16 (round to nearest even) when handed to the GPU; the oracle
reads those same bf16 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WAVE8_TEXT = (445, 349, 293, 185, 202, 82, 97, 71)
CFG_NEG_TEXT = 64   # tokens of a short negative prompt (the pages give no length)
WAVE8_REFS = (0, 4, 3, 4, 2, 3, 4, 3)


@dataclass
class Workload:
    name: str
    seed: int
    n_heads: int
    head_dim: int
    requests: list                 # list of block-length lists [text, refs..., image]
    kv_dtype: str = "bf16"         # prefix cache element type: "bf16", "fp8" or "fp8_v"
    steps: int = 40                # denoising steps per request
    layers: int = 32               # DiT layers (each has its own cache)
    note: str = ""

    @property
    def n_refs(self):
        return [len(bl) - 2 for bl in self.requests]

    @property
    def prefix_lens(self):
        return [int(sum(bl[:-1])) for bl in self.requests]

    @property
    def image_lens(self):
        return [int(bl[-1]) for bl in self.requests]

    @property
    def total_lens(self):
        return [int(sum(bl)) for bl in self.requests]


def _wave8_requests():
    return [[t] + [4096] * r + [4096] for t, r in zip(WAVE8_TEXT, WAVE8_REFS)]


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 64, [[32, 64, 64]], steps=3, layers=1,
                     note="1 head x 64; text 32, one 8x8 reference, 8x8 image latent"),
    "t2i1024": Workload("t2i1024", 1, 24, 128, [[256, 4096]],
                        note="1024x1024 text-to-image, 64x64 latent"),
    "edit4": Workload("edit4", 2, 24, 128, [[256, 4096, 4096, 4096, 4096, 4096]],
                      note="1024x1024 edit with four references"),
    "edit2048": Workload("edit2048", 3, 24, 128, [[512, 4096, 16384]],
                         note="2048x2048 edit with one reference, 128x128 latent"),
    "wave8": Workload("wave8", 4, 24, 128, _wave8_requests(), kv_dtype="fp8",
                      note="eight 1024x1024 requests at one phase, fp8 prefix cache"),
    "edit1": Workload("edit1", 7, 24, 128, [[256, 4096, 4096]],
                      note="1024x1024 edit with one reference"),
    # true CFG: the negative-prompt branch is a second request of the wave with its own
    # (shorter) text, the same reference and an image block of the same size
    "cfg_edit1": Workload("cfg_edit1", 6, 24, 128, [[256, 4096, 4096], [CFG_NEG_TEXT, 4096, 4096]],
                          note="1024x1024 edit with one reference under true CFG: positive "
                               "and negative branch in one wave"),
    "edit10": Workload("edit10", 5, 24, 128, [[256] + [4096] * 10 + [4096]],
                       note="1024x1024 edit with ten references (the model's maximum), "
                            "41,216 prefix tokens"),
}


def rms_rows(rng, n_tokens, gamma):
    """[n_tokens, H, D] float32 rows: N(0,1), unit RMS per (token, head), times gamma."""
    nh, d = gamma.shape
    x = rng.standard_normal((n_tokens, nh, d), dtype=np.float32)
    x /= np.sqrt(np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32))
    x *= gamma[None]
    return x


@dataclass
class WaveInputs:
    """Packed token-major float32 arrays; requests contiguous in wave order."""
    workload: Workload
    q_pre: np.ndarray
    k_pre: np.ndarray
    v_pre: np.ndarray
    q_img: list = field(default_factory=list)   # per step: [sum N_img, H, D]
    k_img: list = field(default_factory=list)
    v_img: list = field(default_factory=list)

    def full(self, step):
        """Packed full-sequence Q, K, V for a step: per request prefix then image rows."""
        w = self.workload
        outs = []
        for pre, img in ((self.q_pre, self.q_img[step]), (self.k_pre, self.k_img[step]),
                         (self.v_pre, self.v_img[step])):
            parts, po, io = [], 0, 0
            for lp, ni in zip(w.prefix_lens, w.image_lens):
                parts.append(pre[po:po + lp])
                parts.append(img[io:io + ni])
                po += lp
                io += ni
            outs.append(np.concatenate(parts, 0))
        return outs


def head_shard(workload, heads=3, requests=None):
    """One GPU's share of a workload under head (tensor or Ulysses) parallelism: the same
    blocks with `heads` of its heads (3 of 24 on eight GPUs; vLLM recipe
    "Qwen/Qwen-Image-2.1", section "Overview"), optionally only some of its requests
    (indices).  Named "<name>@h<heads>"; drawn with the workload's seed."""
    import dataclasses
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    reqs = w.requests if requests is None else [w.requests[i] for i in requests]
    tag = "" if requests is None else "r" + "-".join(map(str, requests))
    return dataclasses.replace(w, name="%s@h%d%s" % (w.name, heads, tag), n_heads=heads,
                               requests=[list(b) for b in reqs])


def workload(name):
    """A workload by name: a key of WORKLOADS, or "<key>@h<n>" for its n-head shard."""
    base, _, heads = name.partition("@h")
    return head_shard(base, int(heads)) if heads else WORKLOADS[base]


def generate(workload, steps=1, seed=None):
    """Draw a wave's inputs for `steps` denoising steps (see module docstring)."""
    w = globals()["workload"](workload) if isinstance(workload, str) else workload
    rng = np.random.default_rng(w.seed if seed is None else seed)
    gam = [rng.uniform(0.8, 1.2, (w.n_heads, w.head_dim)).astype(np.float32)
           for _ in range(3)]
    pre = [[], [], []]
    for lp in w.prefix_lens:
        for t in range(3):
            pre[t].append(rms_rows(rng, lp, gam[t]))
    out = WaveInputs(w, *[np.concatenate(p, 0) if p else
                          np.zeros((0, w.n_heads, w.head_dim), np.float32) for p in pre])
    for _ in range(steps):
        img = [[], [], []]
        for ni in w.image_lens:
            for t in range(3):
                img[t].append(rms_rows(rng, ni, gam[t]))
        out.q_img.append(np.concatenate(img[0], 0))
        out.k_img.append(np.concatenate(img[1], 0))
        out.v_img.append(np.concatenate(img[2], 0))
    return out


def cfg_pair(x: WaveInputs, neg_text=CFG_NEG_TEXT, seed=0):
    """True-CFG wave from a one-request wave x (the positive branch): request 1 is the
    negative branch with a freshly drawn text block of neg_text tokens, the same reference
    blocks and the same image Q/K/V (the two branches see the same latents)."""
    w = x.workload
    assert len(w.requests) == 1
    bl = list(w.requests[0])
    nbl = [int(neg_text)] + bl[1:]
    rng = np.random.default_rng(seed)
    gam = rng.uniform(0.8, 1.2, (w.n_heads, w.head_dim)).astype(np.float32)
    t0 = bl[0]
    pre = []
    for a in (x.q_pre, x.k_pre, x.v_pre):
        neg = np.concatenate([rms_rows(rng, neg_text, gam), a[t0:]], 0)
        pre.append(np.concatenate([a, neg], 0))
    w2 = Workload(w.name + "+cfg", w.seed, w.n_heads, w.head_dim, [bl, nbl], kv_dtype=w.kv_dtype,
                  steps=w.steps, layers=w.layers, note="true-CFG pair")
    out = WaveInputs(w2, *pre)
    for s in range(len(x.q_img)):
        out.q_img.append(np.concatenate([x.q_img[s], x.q_img[s]], 0))
        out.k_img.append(np.concatenate([x.k_img[s], x.k_img[s]], 0))
        out.v_img.append(np.concatenate([x.v_img[s], x.v_img[s]], 0))
    return out


def custom(requests, n_heads, head_dim, kv_dtype="bf16", seed=0, steps=1):
    """Inputs for an arbitrary wave (tests: ragged blocks, edge cases)."""
    w = Workload("custom", seed, n_heads, head_dim, [list(map(int, b)) for b in requests],
                 kv_dtype=kv_dtype, steps=steps, layers=1)
    return generate(w, steps=steps)


def to_bf16(x, device=None):
    """float32 numpy -> torch bf16 tensor (round to nearest even), optionally on device."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t if device is None else t.to(device)


def bf16_exact(x):
    """The float64 values of x after rounding to bf16 (what the GPU actually reads)."""
    import torch
    return to_bf16(x).to(torch.float64).numpy()
