"""fp64 block-causal attention with an explicit mask (test infrastructure only).

What the method computes.  Qwen-Image-2.1's DiT uses block-causal attention over a
sequence made of a text-instruction block, then the reference-image blocks in the order
they were given, then the image-latent block ([blog] "What is Qwen-Image-2.1" table and
"Serving architecture: the cross-step prefix KV cache"; [recipe] "Offline inference":
references are tagged in order).  Because the prefix (text + references) never attends to
the image block, its K/V is identical at every denoising step, so the K/V computed at the
first step can be cached and reused exactly at the later steps ([blog] "Serving
architecture"; [recipe] "Prefix KV cache": exact, not approximate; rebuilt per request).

Readings where the pages are silent (each is listed in the design notes):
  * inside a block attention is bidirectional; between blocks it is causal:
    allowed(q, k)  <=>  blk(k) <= blk(q)                      (plainest meaning of
    "block-causal"; reference i therefore sees text, references 1..i, and itself)
  * softmax scale 1/sqrt(D); no positional term (rotary embedding and Q/K norm are
    upstream of attention, so the inputs stand for post-norm rows)
  * token order: text, ref_1 .. ref_R, image.

Everything is float64, computed from the exact values of the stored inputs (bf16 inputs
widen exactly).  No tiling, blocking or reordering beyond the definition: for every row,
scores over all keys, -inf where the mask forbids, subtract the row max over the allowed
keys, exponentiate, normalise, multiply by V.  Work is split per head and into row chunks
only to bound memory; each row is computed independently, so this changes nothing.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024  # rows per explicit-mask chunk; memory bound only


def block_offsets(block_len):
    """o_0 = 0, o_{b+1} = o_b + l_b.  Returns int64 array of length n_blocks + 1."""
    bl = np.asarray(block_len, dtype=np.int64)
    if bl.ndim != 1 or bl.size == 0 or np.any(bl <= 0):
        raise ValueError("block lengths must be a non-empty list of positive integers")
    return np.concatenate([[0], np.cumsum(bl)])


def block_of_position(block_len):
    """blk(p) for every position p of one request: index of the block holding p."""
    bl = np.asarray(block_len, dtype=np.int64)
    return np.repeat(np.arange(bl.size, dtype=np.int64), bl)


def allowed_mask(block_len, rows=None, keys=None):
    """Explicit boolean mask allowed[q, k] = blk(k) <= blk(q) for one request.

    rows / keys select position ranges (python ranges or index arrays); default all.
    """
    blk = block_of_position(block_len)
    r = np.arange(blk.size) if rows is None else np.asarray(rows, dtype=np.int64)
    k = np.arange(blk.size) if keys is None else np.asarray(keys, dtype=np.int64)
    return blk[k][None, :] <= blk[r][:, None]


def masked_attention_head(q, k, v, allowed, scale):
    """softmax_k(q k^T * scale, -inf where not allowed) v for one head, in float64.

    q [Nq, D], k [Nk, D], v [Nk, Dv], allowed bool [Nq, Nk].  Every row must have at
    least one allowed key (the method guarantees it: each row sees its own block).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if not np.all(allowed.any(axis=1)):
        raise ValueError("a row with no allowed key has no softmax")
    s = (q @ k.T) * scale
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def masked_attention(q, k, v, allowed, scale=None):
    """Multi-head wrapper.  q [Nq, H, D], k/v [Nk, H, D], allowed [Nq, Nk] -> [Nq, H, D]."""
    q = np.asarray(q)
    nq, nh, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.empty((nq, nh, v.shape[2]), dtype=np.float64)
    for h in range(nh):
        kh = np.asarray(k[:, h, :], dtype=np.float64)
        vh = np.asarray(v[:, h, :], dtype=np.float64)
        for r0 in range(0, nq, ROW_CHUNK):
            r1 = min(nq, r0 + ROW_CHUNK)
            out[r0:r1, h, :] = masked_attention_head(q[r0:r1, h, :], kh, vh,
                                                     allowed[r0:r1], scale)
    return out


# --------------------------------------------------------------------------------------
# The three calls of the hot path, for ONE request.  block_len = [text, ref_1..ref_R,
# image]; the prefix is every block but the last.
# --------------------------------------------------------------------------------------

def prefix_length(block_len):
    return int(np.sum(block_len[:-1]))


def full_step(block_len, q_all, k_all, v_all, scale=None):
    """Full recompute: all N rows over all N keys, block-causal.  [N, H, D] each."""
    n = int(np.sum(block_len))
    if q_all.shape[0] != n or k_all.shape[0] != n or v_all.shape[0] != n:
        raise ValueError("full-step tensors must hold N tokens")
    return masked_attention(q_all, k_all, v_all, allowed_mask(block_len), scale)


def prefix_step(block_len, q_pre, k_pre, v_pre, scale=None):
    """Step-0 prefix attention: prefix rows over prefix keys, block-causal.

    The prefix rows never see the image block, so this is the full step restricted to
    the prefix (the reason its K/V can be cached: [blog] "Serving architecture").
    """
    lp = prefix_length(block_len)
    if lp == 0:
        return np.zeros((0,) + tuple(q_pre.shape[1:]), dtype=np.float64)
    return masked_attention(q_pre, k_pre, v_pre, allowed_mask(block_len[:-1]), scale)


def denoise_step(block_len, q_img, k_pre, v_pre, k_img, v_img, scale=None):
    """Denoising-step attention: image rows over [cached prefix keys ; live image keys].

    k_pre / v_pre are whatever the cache holds (exact bf16 values, or the dequantised
    fp8 values code * scale); the image block sees every key of its request.
    """
    lp = prefix_length(block_len)
    n = int(np.sum(block_len))
    k = np.concatenate([np.asarray(k_pre, np.float64), np.asarray(k_img, np.float64)], 0)
    v = np.concatenate([np.asarray(v_pre, np.float64), np.asarray(v_img, np.float64)], 0)
    if k.shape[0] != n or q_img.shape[0] != n - lp:
        raise ValueError("denoise tensors do not match the block lengths")
    return masked_attention(q_img, k, v, allowed_mask(block_len, rows=range(lp, n)), scale)
