"""Pins for the fp64 attention oracle (CPU only).

Each test checks oracle/attention.py against something other than itself: a pure-Python
brute force on the tiny workload, torch's scaled_dot_product_attention in the special
cases where block-causal attention reduces to it, closed forms, and invariants that the
block-causal structure fixes.  A plausible mistake (dropped scale, mask transposed or off
by one block, wrong softmax axis, wrong normalisation, swapped K/V) fails at least one.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from block_causal_attention_qi_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ---------------------------------------------------------------- brute force (tiny)

def _brute_block_index(block_len, p):
    start = 0
    for b, length in enumerate(block_len):
        if start <= p < start + length:
            return b
        start += length
    raise IndexError(p)


def _brute_attention(block_len, rows, q, k, v):
    """Scalar loops, math.exp, log-sum-exp normalisation.  q: list over rows, k/v over keys
    (keys are positions 0..len(k)-1 of the request); one head."""
    d = len(q[0])
    out = []
    for qi, p in zip(q, rows):
        bq = _brute_block_index(block_len, p)
        logits = []
        for kk in range(len(k)):
            if _brute_block_index(block_len, kk) <= bq:
                dot = 0.0
                for c in range(d):
                    dot += qi[c] * k[kk][c]
                logits.append((kk, dot / math.sqrt(d)))
        mx = max(val for _, val in logits)
        lse = mx + math.log(sum(math.exp(val - mx) for _, val in logits))
        row = [0.0] * len(v[0])
        for kk, val in logits:
            w = math.exp(val - lse)
            for c in range(len(row)):
                row[c] += w * v[kk][c]
        out.append(row)
    return np.array(out)


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS["tiny"]
    return w, synth.generate(w, steps=3)


def test_brute_force_tiny_all_calls(tiny):
    w, x = tiny
    bl = w.requests[0]
    lp = w.prefix_lens[0]
    qp, kp, vp = (synth.bf16_exact(t) for t in (x.q_pre, x.k_pre, x.v_pre))
    # prefix build (step 0)
    got = A.prefix_step(bl, qp, kp, vp)[:, 0, :]
    ref = _brute_attention(bl, range(lp), qp[:, 0].tolist(), kp[:, 0].tolist(), vp[:, 0].tolist())
    assert np.max(np.abs(got - ref)) <= 1e-12
    for s in range(3):
        qi, ki, vi = (synth.bf16_exact(t[s]) for t in (x.q_img, x.k_img, x.v_img))
        got = A.denoise_step(bl, qi, kp, vp, ki, vi)[:, 0, :]
        kall = np.concatenate([kp, ki])[:, 0].tolist()
        vall = np.concatenate([vp, vi])[:, 0].tolist()
        ref = _brute_attention(bl, range(lp, lp + len(qi)), qi[:, 0].tolist(), kall, vall)
        assert np.max(np.abs(got - ref)) <= 1e-12, s
    qa, ka, va = (synth.bf16_exact(t) for t in x.full(0))
    got = A.full_step(bl, qa, ka, va)[:, 0, :]
    ref = _brute_attention(bl, range(len(qa)), qa[:, 0].tolist(), ka[:, 0].tolist(), va[:, 0].tolist())
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_brute_force_tiny_float32_rows(tiny):
    """The tiny case as drawn, in float32 (widened exactly to float64), before any rounding
    to bf16: the full step and the last denoising step against the brute force."""
    w, x = tiny
    bl = w.requests[0]
    lp = w.prefix_lens[0]
    qa, ka, va = (np.asarray(t, dtype=np.float64) for t in x.full(2))
    assert x.q_pre.dtype == np.float32
    got = A.full_step(bl, qa, ka, va)[:, 0, :]
    ref = _brute_attention(bl, range(len(qa)), qa[:, 0].tolist(), ka[:, 0].tolist(), va[:, 0].tolist())
    assert np.max(np.abs(got - ref)) <= 1e-12
    got = A.denoise_step(bl, qa[lp:], ka[:lp], va[:lp], ka[lp:], va[lp:])[:, 0, :]
    assert np.max(np.abs(got - ref[lp:])) <= 1e-12


# ---------------------------------------------------------------- library special cases

def _sdpa(q, k, v, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.transpose(a, (1, 0, 2))))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    return np.transpose(o.numpy(), (1, 0, 2))


def test_unit_blocks_equal_token_causal_sdpa():
    rng = np.random.default_rng(11)
    n, h, d = 37, 3, 16
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    got = A.full_step([1] * n, q, k, v)
    assert np.max(np.abs(got - _sdpa(q, k, v, True))) < 1e-12


def test_single_block_equals_unmasked_sdpa():
    rng = np.random.default_rng(12)
    n, h, d = 29, 2, 32
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    assert np.max(np.abs(A.full_step([n], q, k, v) - _sdpa(q, k, v, False))) < 1e-12


def test_denoise_equals_unmasked_sdpa_over_all_keys():
    rng = np.random.default_rng(13)
    bl = [5, 7, 3, 9]
    lp, n, h, d = 15, 24, 2, 8
    k, v = rng.standard_normal((n, h, d)), rng.standard_normal((n, h, d))
    qi = rng.standard_normal((n - lp, h, d))
    got = A.denoise_step(bl, qi, k[:lp], v[:lp], k[lp:], v[lp:])
    ref = np.transpose(torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.transpose(qi, (1, 0, 2)).copy()),
        torch.from_numpy(np.transpose(k, (1, 0, 2)).copy()),
        torch.from_numpy(np.transpose(v, (1, 0, 2)).copy())).numpy(), (1, 0, 2))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_block_causal_equals_sdpa_with_block_mask():
    """Independent mask built from block boundaries by set membership, fed to SDPA."""
    rng = np.random.default_rng(14)
    bl = [4, 6, 6, 5]
    n, h, d = sum(bl), 2, 8
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    ends = np.cumsum(bl)
    m = np.zeros((n, n), dtype=bool)
    for qpos in range(n):
        visible_end = int(ends[np.searchsorted(ends, qpos, side="right")])
        m[qpos, :visible_end] = True
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.transpose(a, (1, 0, 2))))
    ref = np.transpose(torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(m)).numpy(), (1, 0, 2))
    assert np.max(np.abs(A.full_step(bl, q, k, v) - ref)) < 1e-12


# ---------------------------------------------------------------- closed forms

def test_constant_keys_give_mean_of_allowed_values():
    rng = np.random.default_rng(15)
    bl = [3, 5, 4, 6]
    n, h, d = sum(bl), 2, 8
    q, v = rng.standard_normal((n, h, d)), rng.standard_normal((n, h, d))
    k = np.broadcast_to(rng.standard_normal((1, h, d)), (n, h, d)).copy()
    got = A.full_step(bl, q, k, v)
    ends = np.cumsum(bl)
    for p in range(n):
        e = int(ends[np.searchsorted(ends, p, side="right")])
        assert np.allclose(got[p], v[:e].mean(axis=0), atol=1e-13, rtol=0)


def test_unit_values_give_unit_output():
    rng = np.random.default_rng(16)
    bl = [7, 9, 5]
    n, h, d = sum(bl), 3, 8
    q, k = rng.standard_normal((n, h, d)) * 3, rng.standard_normal((n, h, d)) * 3
    got = A.full_step(bl, q, k, np.ones((n, h, d)))
    assert np.max(np.abs(got - 1.0)) < 1e-14


def test_one_hot_values_recover_probabilities(tiny):
    """V = one-hot slices (3 passes of 64 keys at D=64) recover P: rows sum to 1, P is
    exactly 0 on forbidden pairs and positive on allowed ones, and P matches exp/sum."""
    w, x = tiny
    bl = w.requests[0]
    qa, ka, _ = (synth.bf16_exact(t) for t in x.full(0))
    n, d = qa.shape[0], qa.shape[2]
    p = np.zeros((n, n))
    for k0 in range(0, n, d):
        k1 = min(n, k0 + d)
        v = np.zeros((n, 1, d))
        v[np.arange(k0, k1), 0, np.arange(k1 - k0)] = 1.0
        p[:, k0:k1] = A.full_step(bl, qa, ka, v)[:, 0, :k1 - k0]
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) < 1e-13
    blk = np.repeat(np.arange(len(bl)), bl)
    forbidden = blk[None, :] > blk[:, None]
    assert np.all(p[forbidden] == 0.0)
    assert np.all(p[~forbidden] > 0.0)
    # explicit probabilities for one row of each block
    for row in (0, 40, 150):
        allowed = ~forbidden[row]
        s = (ka[allowed, 0] @ qa[row, 0]) / math.sqrt(d)
        e = np.exp(s - s.max())
        assert np.allclose(p[row, allowed], e / e.sum(), atol=1e-14, rtol=0)


def test_scale_is_inverse_sqrt_head_dim():
    """Two keys, one query: the softmax weight ratio must be exp((s1 - s2) / sqrt(D))."""
    d = 16
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 4.0
    k = np.zeros((2, 1, d)); k[0, 0, 0] = 1.0; k[1, 0, 0] = -1.0
    v = np.zeros((2, 1, d)); v[0, 0, 0] = 1.0; v[1, 0, 1] = 1.0
    out = A.masked_attention(q, k, v, np.ones((1, 2), bool))[0, 0]
    assert math.isclose(out[0] / out[1], math.exp(8.0 / math.sqrt(d)), rel_tol=1e-13)


# ---------------------------------------------------------------- invariants

def test_prefix_rows_do_not_depend_on_image_tokens():
    rng = np.random.default_rng(17)
    bl = [6, 10, 10, 12]
    n, h, d = sum(bl), 2, 16
    lp = n - bl[-1]
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    a = A.full_step(bl, q, k, v)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for t in (q2, k2, v2):
        t[lp:] = rng.standard_normal((n - lp, h, d)) * 5
    b = A.full_step(bl, q2, k2, v2)
    assert np.array_equal(a[:lp], b[:lp])
    assert not np.allclose(a[lp:], b[lp:])


def test_reuse_equals_full_recompute():
    rng = np.random.default_rng(18)
    bl = [6, 10, 10, 12]
    n, h, d = sum(bl), 2, 16
    lp = n - bl[-1]
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    full = A.full_step(bl, q, k, v)
    pre = A.prefix_step(bl, q[:lp], k[:lp], v[:lp])
    den = A.denoise_step(bl, q[lp:], k[:lp], v[:lp], k[lp:], v[lp:])
    assert np.max(np.abs(full[:lp] - pre)) < 1e-14
    assert np.max(np.abs(full[lp:] - den)) < 1e-14


def test_references_see_only_earlier_references():
    """Changing reference 2 changes rows of refs 2..R and the image, never text or ref 1."""
    rng = np.random.default_rng(19)
    bl = [4, 5, 5, 5, 6]
    n, h, d = sum(bl), 1, 8
    q, k, v = (rng.standard_normal((n, h, d)) for _ in range(3))
    a = A.full_step(bl, q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[9:14] += 1.0
    v2[9:14] += 1.0
    b = A.full_step(bl, q, k2, v2)
    assert np.array_equal(a[:9], b[:9])
    assert np.all(np.abs(a[9:] - b[9:]).max(axis=(1, 2)) > 0)


def test_rejects_empty_blocks_and_bad_shapes():
    with pytest.raises(ValueError):
        A.block_offsets([3, 0, 2])
    with pytest.raises(ValueError):
        A.full_step([2, 2], np.zeros((3, 1, 4)), np.zeros((4, 1, 4)), np.zeros((4, 1, 4)))
