"""Prefix-cache byte layout, tile classification map and useful-pair counts
(test infrastructure only).

None of these is given by the pages; they are this library's own definitions, written out
plainly here so that the library's host code can be checked against them bit for bit.

Cache layout (one arena per layer and wave; [recipe] "Prefix KV cache" says the cache is
rebuilt for every generation, so it holds exactly the requests of one wave):
  requests follow one another in wave order; each request's region starts on a 256-byte
  boundary and holds, each part again starting on a 256-byte boundary,
      K  [H][L_p][D]   bf16 (2 bytes), or E4M3FN code (1 byte) for the "fp8" cache
      V  [H][L_p][D]   bf16, or E4M3FN code for the "fp8" and "fp8_v" caches
      scales [2][H]    float32, row 0 for K and row 1 for V  (fp8 caches only; the
                       "fp8_v" cache keeps K in bf16 and stores 1.0 as its K scales)
  the arena size is the end of the last region rounded up to 256 bytes.

Tiling (what the attention kernels launch over):
  * calls: PREFIX = prefix rows over prefix keys (step 0); DENOISE = image rows over all
    keys; FULL = all rows over all keys.
  * row tiles never cross a block: each block of the call's row set is cut into tiles of
    bm rows starting at the block's first row (the last tile of a block may be short);
  * key tiles start at key 0 of the request and hold bn keys (the last may be short);
  * class of a tile (row tile x key tile), from the explicit block-causal mask:
    EMPTY (0) no allowed pair, PARTIAL (1) some, FULL (2) all.
  The map is laid out request by request, row tile by row tile, key tile by key tile.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_mask, block_offsets

ALIGN = 256
EMPTY, PARTIAL, FULL = 0, 1, 2
CALL_PREFIX, CALL_DENOISE, CALL_FULL = 0, 1, 2
KV_BF16, KV_FP8, KV_FP8_V = 0, 1, 2


def _elem_bytes(kv_dtype, which):
    """Bytes per cached element of K (which = 0) or V (which = 1)."""
    if kv_dtype == KV_BF16:
        return 2
    if kv_dtype == KV_FP8:
        return 1
    if kv_dtype == KV_FP8_V:
        return 2 if which == 0 else 1
    raise ValueError("unknown cache type")


def _align(x):
    return (x + ALIGN - 1) // ALIGN * ALIGN


def cache_layout(requests, n_heads, head_dim, kv_dtype):
    """requests: list of block-length lists.  Returns (regions, total_bytes)."""
    ek, ev = _elem_bytes(kv_dtype, 0), _elem_bytes(kv_dtype, 1)
    regions, off = [], 0
    for bl in requests:
        lp = int(np.sum(bl[:-1]))
        start = _align(off)
        k_off = start
        v_off = _align(k_off + n_heads * lp * head_dim * ek)
        end = v_off + n_heads * lp * head_dim * ev
        s_off = None
        if kv_dtype != KV_BF16:
            s_off = _align(end)
            end = s_off + 2 * n_heads * 4
        regions.append(dict(lp=lp, k_off=k_off, v_off=v_off, s_off=s_off, end=end))
        off = end
    return regions, _align(off)


def cache_offset(regions, head_dim, kv_dtype, req, kv, head, tok):
    """Byte offset of element (req, K|V, head, token, channel 0) in the arena."""
    eb = _elem_bytes(kv_dtype, kv)
    reg = regions[req]
    base = reg["k_off"] if kv == 0 else reg["v_off"]
    return base + (head * reg["lp"] + tok) * head_dim * eb


def bf16_bits(values):
    """uint16 bit patterns of values that are exactly representable in bf16."""
    f32 = np.ascontiguousarray(values, dtype=np.float32)
    if not np.array_equal(f32.astype(np.float64), np.asarray(values, dtype=np.float64)):
        raise ValueError("values are not bf16-exact")
    bits = f32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (bits >> 16).astype(np.uint16)


def cache_image(requests, n_heads, head_dim, kv_dtype, k_pre, v_pre):
    """Expected bytes of the cache arena after the prefix build.

    k_pre / v_pre: packed token-major [sum L_p, H, D] bf16-exact values of the wave.
    Returns (image uint8 [total], defined bool [total]); padding bytes are undefined.
    """
    from . import fp8 as F
    regions, total = cache_layout(requests, n_heads, head_dim, kv_dtype)
    img = np.zeros(total, dtype=np.uint8)
    defined = np.zeros(total, dtype=bool)
    tok = 0
    for reg in regions:
        lp = reg["lp"]
        kr = np.asarray(k_pre[tok:tok + lp], dtype=np.float64)
        vr = np.asarray(v_pre[tok:tok + lp], dtype=np.float64)
        tok += lp
        if kv_dtype == KV_BF16:
            parts = [(reg["k_off"], bf16_bits(np.transpose(kr, (1, 0, 2))).view(np.uint8)),
                     (reg["v_off"], bf16_bits(np.transpose(vr, (1, 0, 2))).view(np.uint8))]
        elif kv_dtype == KV_FP8:
            ck, cv, sc = F.quantize_prefix(kr, vr)
            parts = [(reg["k_off"], ck), (reg["v_off"], cv),
                     (reg["s_off"], sc.astype("<f4").view(np.uint8))]
        else:
            cv, sv = F.quantize_prefix_v(vr)
            sc = np.stack([np.ones_like(sv), sv])
            parts = [(reg["k_off"], bf16_bits(np.transpose(kr, (1, 0, 2))).view(np.uint8)),
                     (reg["v_off"], cv), (reg["s_off"], sc.astype("<f4").view(np.uint8))]
        for off, arr in parts:
            flat = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
            img[off:off + flat.size] = flat
            defined[off:off + flat.size] = True
    return img, defined


def call_rows_keys(block_len, call):
    """(row blocks, key count) of one request for a call.  Row blocks are (start, len)."""
    off = block_offsets(block_len)
    nb = len(block_len)
    if call == CALL_PREFIX:
        blocks = range(0, nb - 1)
        nkeys = int(off[nb - 1])
    elif call == CALL_DENOISE:
        blocks = range(nb - 1, nb)
        nkeys = int(off[nb])
    elif call == CALL_FULL:
        blocks = range(0, nb)
        nkeys = int(off[nb])
    else:
        raise ValueError("unknown call")
    return [(int(off[b]), int(block_len[b])) for b in blocks], nkeys


def row_tiles(block_len, call, bm):
    """List of (first row, row count) for the call's row tiles of one request."""
    tiles = []
    for start, length in call_rows_keys(block_len, call)[0]:
        for r0 in range(start, start + length, bm):
            tiles.append((r0, min(bm, start + length - r0)))
    return tiles


def tile_map(block_len, call, bm, bn):
    """uint8 [n_row_tiles, n_key_tiles] for one request, classified from the explicit mask."""
    _, nkeys = call_rows_keys(block_len, call)
    rt = row_tiles(block_len, call, bm)
    nkt = (nkeys + bn - 1) // bn
    out = np.empty((len(rt), nkt), dtype=np.uint8)
    for i, (r0, nr) in enumerate(rt):
        rows_mask = allowed_mask(block_len, rows=range(r0, r0 + nr), keys=range(nkeys))
        for j in range(nkt):
            sub = rows_mask[:, j * bn:min(nkeys, (j + 1) * bn)]
            out[i, j] = FULL if sub.all() else (EMPTY if not sub.any() else PARTIAL)
    return out


def wave_tile_map(requests, call, bm, bn):
    """Concatenation of tile_map over the wave's requests, flattened."""
    return np.concatenate([tile_map(bl, call, bm, bn).ravel() for bl in requests])


def useful_pairs(block_len, call):
    """Number of allowed (row, key) pairs the call computes for one request."""
    blocks, nkeys = call_rows_keys(block_len, call)
    total = 0
    for start, length in blocks:
        for r0 in range(start, start + length, 1024):   # row chunks bound memory only
            r1 = min(start + length, r0 + 1024)
            total += int(allowed_mask(block_len, rows=range(r0, r1),
                                      keys=range(nkeys)).sum())
    return total


def useful_flops(requests, call, n_heads, head_dim):
    """4 * D * H * pairs: two multiply-adds per (pair, channel), QK^T and PV."""
    return 4 * head_dim * n_heads * sum(useful_pairs(bl, call) for bl in requests)
