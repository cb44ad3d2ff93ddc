"""FP8 (OCP E4M3FN) prefix-cache quantisation, written from the format's definition
(test infrastructure only).

The pages say the prefix KV cache may be stored in FP8, as "fp8" (K and V) or "fp8_v"
(V only), at some cost in quality and speed ([recipe] "Prefix KV cache").  They fix
neither the FP8 format, nor the scale granularity, nor the rounding.  Readings taken:
  * format: OCP E4M3FN -- sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals when the exponent field is 0, no infinities, S.1111.111 is NaN, largest
    finite magnitude 448 (this is the FP8 flavour gfx950 converts natively);
  * one float32 scale per (request, head, K or V) over all prefix positions and
    channels: a = max |x|, scale = a / 448, inv = 448 / a (each one IEEE float32
    division, correctly rounded); a == 0 gives scale = inv = 1;
  * code = nearest E4M3FN value to the float32 product x * inv, ties to the even
    code, magnitudes at or above 448 saturate to 448 (never NaN);
  * dequantised value = value(code) * scale, exact in float64.

Where floating point decides an integer code, this module takes the decision in float32
like the kernel does (the product x * inv is a float32 multiply); the nearest-value search
itself is exact in float64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3fn_value(code):
    """Exact value of an E4M3FN code (uint8 or int array), float64; NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e.astype(np.float64) - 10))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


# magnitudes of the 127 non-negative finite codes 0x00..0x7E, ascending with the code
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3fn_value(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0) and _POS_VALUES[-1] == E4M3_MAX


def e4m3fn_encode(y):
    """Round float32 values to E4M3FN codes: nearest, ties to even code, saturating."""
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.isnan(y)):
        raise ValueError("NaN has no saturating code")
    a = np.abs(y.astype(np.float64))
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, _POS_CODES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_POS_VALUES[hi] - a)
    d_lo = np.abs(a - _POS_VALUES[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    sign = np.signbit(y).astype(np.int64)
    return ((sign << 7) | code).astype(np.uint8)


def absmax_scale(x):
    """(scale, inv) float32 pair for one slab of values (any shape)."""
    a = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else np.float32(0)
    if a == 0:
        return np.float32(1.0), np.float32(1.0)
    return np.float32(a) / np.float32(E4M3_MAX), np.float32(E4M3_MAX) / np.float32(a)


def quantize_slab(x):
    """Quantise one (request, head, K|V) slab [L_p, D].  Returns (codes uint8, scale f32)."""
    scale, inv = absmax_scale(x)
    y = np.asarray(x, dtype=np.float32) * inv   # float32 multiply, round to nearest even
    return e4m3fn_encode(y), scale


def quantize_prefix(k_pre, v_pre):
    """Quantise a request's prefix K and V, [L_p, H, D] each.

    Returns codes_k [H, L_p, D], codes_v [H, L_p, D] (uint8) and scales [2, H] float32
    (row 0: K, row 1: V), i.e. the cache's own head-major arrangement.
    """
    lp, nh, d = k_pre.shape
    codes = np.empty((2, nh, lp, d), dtype=np.uint8)
    scales = np.empty((2, nh), dtype=np.float32)
    for kv, x in enumerate((k_pre, v_pre)):
        for h in range(nh):
            codes[kv, h], scales[kv, h] = quantize_slab(np.asarray(x)[:, h, :])
    return codes[0], codes[1], scales


def quantize_prefix_v(v_pre):
    """The "fp8_v" cache: V only, [L_p, H, D] -> codes [H, L_p, D] uint8, scales [H]."""
    lp, nh, d = v_pre.shape
    codes = np.empty((nh, lp, d), dtype=np.uint8)
    scales = np.empty(nh, dtype=np.float32)
    for h in range(nh):
        codes[h], scales[h] = quantize_slab(np.asarray(v_pre)[:, h, :])
    return codes, scales


def dequantize(codes_hld, scales_h):
    """codes [H, L_p, D] and scales [H] -> values [L_p, H, D] float64 (token-major)."""
    vals = e4m3fn_value(codes_hld) * np.asarray(scales_h, dtype=np.float64)[:, None, None]
    return np.transpose(vals, (1, 0, 2))
