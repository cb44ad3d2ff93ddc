"""Pins for the fp8 (OCP E4M3FN) quantiser of the oracle (CPU only).

The encoder is checked against torch's float8_e4m3fn conversion (a library routine) over
every bf16 bit pattern in range, against values worked out from the format's definition,
and the per-slab absmax quantisation against its error bound and the absmax identity.
"""
import numpy as np
import pytest
import torch

from oracle import fp8


def _all_bf16_in_range():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    return vals[keep]


def test_encoder_matches_torch_over_all_bf16_values():
    y = _all_bf16_in_range()
    ours = fp8.e4m3fn_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encoder_matches_torch_on_float32_ties_and_near_ties():
    rng = np.random.default_rng(3)
    vals = fp8._POS_VALUES[1:]
    mids = (vals[:-1] + vals[1:]) / 2          # exact ties between neighbours
    y = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    y = np.concatenate([y, -y])
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3fn_encode(y), ref)


def test_codes_from_the_format_definition():
    cases = {
        1.0: 0x38,            # exponent field 7 (bias 7), mantissa 0
        -1.0: 0xB8,
        2.0 ** -9: 0x01,      # smallest subnormal
        2.0 ** -6: 0x08,      # smallest normal
        0.5 * 2 ** -9: 0x00,  # tie between 0 and 2^-9 -> even code 0
        1.5 * 2 ** -9: 0x02,  # tie between codes 1 and 2 -> even
        1.0625: 0x38,         # tie between 1.0 (0x38) and 1.125 (0x39) -> even
        1.1875: 0x3A,         # tie between 1.125 (0x39) and 1.25 (0x3A) -> even
        240.0: 0x77,          # 1.875 * 2^7
        256.0: 0x78,          # exponent field 15, mantissa 0 is a finite number
        448.0: 0x7E,          # largest finite
        460.0: 0x7E,          # saturates, never NaN
        1e6: 0x7E,
        -1e6: 0xFE,
        0.0: 0x00,
    }
    y = np.array(list(cases) + [-0.0], dtype=np.float32)   # -0.0 keeps its sign bit
    assert list(fp8.e4m3fn_encode(y)) == list(cases.values()) + [0x80]


def test_value_table_matches_torch_decode():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.e4m3fn_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}


def test_absmax_quantisation_bounds():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 64)) * 0.7).astype(np.float32)
    x[17, 3] = -5.0                      # the absmax element (others are below 4)
    codes, scale = fp8.quantize_slab(x)
    assert np.abs(x).max() == 5.0 and scale == np.float32(5.0) / np.float32(448)
    assert codes[17, 3] == 0xFE          # -448 exactly
    deq = fp8.e4m3fn_value(codes) * np.float64(scale)
    normal = np.abs(x) >= 2.0 ** -6 * float(scale)
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)          # 3 mantissa bits, round to nearest
    assert np.abs(deq - x)[~normal].max(initial=0) <= 2.0 ** -10 * float(scale) * (1 + 1e-6)


def test_zero_slab_has_unit_scale():
    codes, scale = fp8.quantize_slab(np.zeros((5, 8), np.float32))
    assert scale == 1.0 and not codes.any()


def test_quantize_prefix_shapes_and_roundtrip():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((40, 3, 16)).astype(np.float32)
    v = rng.standard_normal((40, 3, 16)).astype(np.float32) * 3
    ck, cv, sc = fp8.quantize_prefix(k, v)
    assert ck.shape == (3, 40, 16) and cv.shape == (3, 40, 16) and sc.shape == (2, 3)
    for h in range(3):
        assert sc[0, h] == np.float32(np.abs(k[:, h]).max()) / np.float32(448)
        assert sc[1, h] == np.float32(np.abs(v[:, h]).max()) / np.float32(448)
    dk = fp8.dequantize(ck, sc[0])
    assert dk.shape == k.shape
    assert np.max(np.abs(dk - k) / np.maximum(np.abs(k), 1e-3)) < 0.07


def test_encoder_rejects_nan():
    with pytest.raises(ValueError):
        fp8.e4m3fn_encode(np.array([np.nan], np.float32))


def test_v_only_quantisation_is_the_v_half():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((37, 3, 16)) * 3
    v = rng.standard_normal((37, 3, 16)) * 0.01
    ck, cv, sc = fp8.quantize_prefix(k, v)
    cv2, sv = fp8.quantize_prefix_v(v)
    assert np.array_equal(cv, cv2) and np.array_equal(sc[1], sv)
