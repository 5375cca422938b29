"""The oracle's E4M3 format against torch's float8_e4m3fn and the format's fixed points."""
import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.DECODE_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(want))
    m = ~np.isnan(want)
    assert np.array_equal(got[m], want[m])


def test_format_fixed_points():
    assert fp8.decode_code(0x7E) == 448.0 and fp8.decode_code(0xFE) == -448.0
    assert fp8.decode_code(0x38) == 1.0
    assert fp8.decode_code(0x08) == 2.0 ** -6          # smallest normal
    assert fp8.decode_code(0x01) == 2.0 ** -9          # smallest subnormal
    assert fp8.decode_code(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert math.isnan(fp8.decode_code(0x7F)) and math.isnan(fp8.decode_code(0xFF))
    assert fp8.decode_code(0x00) == 0.0 and math.copysign(1, fp8.decode_code(0x80)) < 0
    assert int(np.sum(np.isnan(fp8.DECODE_TABLE))) == 2   # no infinities, two NaNs


def test_encode_round_trips_every_finite_code():
    for c in range(256):
        v = fp8.decode_code(c)
        if not math.isnan(v):
            assert fp8.encode_value(v) == c, hex(c)


def test_encode_ties_go_to_even_code():
    vals = fp8.DECODE_TABLE[:0x7F]
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert fp8.encode_value(mid) == want
        assert fp8.encode_value(-mid) == 0x80 | want


def test_encode_saturates_and_keeps_nan():
    assert fp8.encode_value(448.0) == 0x7E
    assert fp8.encode_value(460.0) == 0x7E
    assert fp8.encode_value(1e30) == 0x7E and fp8.encode_value(-1e30) == 0xFE
    assert fp8.encode_value(float("inf")) == 0x7E
    assert fp8.encode_value(float("nan")) == 0x7F
    assert fp8.encode_value(2.0 ** -11) == 0x00          # below half the smallest subnormal
    assert fp8.encode_value(-(2.0 ** -11)) == 0x80


def test_vectorized_encode_is_the_scalar_definition():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(3000) * s for s in (1e-4, 0.01, 1.0, 100.0, 1e3)])
    mids = [(fp8.DECODE_TABLE[c] + fp8.DECODE_TABLE[c + 1]) / 2 for c in range(0x7E)]
    x = np.concatenate([x, mids, -np.asarray(mids), fp8.DECODE_TABLE[:0x7F],
                        [0.0, -0.0, np.inf, -np.inf, np.nan, 448.0, 500.0, -1e9]])
    want = np.array([fp8.encode_value(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(fp8.encode(x), want)


def test_encode_matches_torch_in_range():
    g = torch.Generator().manual_seed(0)
    x = torch.cat([torch.randn(20000, generator=g) * s for s in (0.01, 0.3, 3.0, 60.0)])
    x = x[x.abs() < 440].to(torch.float64)
    want = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = fp8.encode(x.numpy())
    assert np.array_equal(got, want)


def test_quantize_with_scale():
    x = np.array([0.5, -3.0, 100.0])
    c = fp8.quantize(x, 0.25)
    np.testing.assert_allclose(fp8.dequantize(c, 0.25), [0.5, -3.0, 100.0], rtol=0.07)


def test_quantize_rows_decides_in_float32():
    """The code comes from float32(x) * float32(1/scale), not from the exact quotient.

    x = float32(25.2) = 25.2000007629..., scale 0.3: the exact quotient 84.0000025 lies
    just above 84, the midpoint of the E4M3 neighbours 80 (code 0x6A) and 88 (0x6B), so
    exact division would give 0x6B; the float32 product rounds to 84.0 exactly, a tie,
    which goes to the even code 0x6A."""
    import torch
    from oracle import cache_ops
    x = torch.tensor([25.2, -25.2], dtype=torch.float32)
    assert fp8.encode_value(float(x[0]) / 0.3) == 0x6B
    assert cache_ops.quantize_rows(x, 0.3).tolist() == [0x6A, 0xEA]


def test_fp8_attention_is_attention_on_dequantized_pools():
    from oracle import attention
    import pins
    rng = np.random.default_rng(3)
    lens = [5, 11]
    q, lk, lv, kc, vc, tables = pins._random_case(31, lens, H=2, Hkv=2, D=8, B=4)
    kq = fp8.quantize(np.nan_to_num(kc), 0.5)
    vq = fp8.quantize(np.nan_to_num(vc), 0.25)
    got = attention.decode_attention(q, kq, vq, tables, lens, 4, k_scale=0.5, v_scale=0.25)
    want = attention.decode_attention(q, fp8.dequantize(kq, 0.5), fp8.dequantize(vq, 0.25),
                                      tables, lens, 4)
    assert np.array_equal(got, want)
