"""Pins for the oracle's e4m3fn codec (CPU only).

The decode table is checked against torch's float8_e4m3fn type (a library
implementation of the same OCP format) and a few hand values; the encoder is
checked bit for bit against torch's cast for every bf16 input that does not
overflow, at eight head scales, and against the saturation reading beyond.
"""

import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_matches_torch_for_all_codes():
    ours = fp8.decode_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)])
    assert np.isnan(ours).sum() == 2                     # 0x7f and 0xff only


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                                        (0x08, 2.0 ** -6), (0x38, 1.0), (0x7E, 448.0),
                                        (0xFE, -448.0), (0x40, 2.0), (0x3C, 1.5)])
def test_decode_hand_values(code, value):
    assert fp8.decode(code) == value


def test_roundtrip_every_finite_code():
    for c in range(256):
        v = fp8.decode(c)
        if math.isnan(v):
            continue
        assert fp8.encode_one(v) == c


def test_saturation_and_nan():
    assert fp8.encode_one(448.0) == 0x7E
    assert fp8.encode_one(463.99) == 0x7E
    assert fp8.encode_one(464.0) == 0x7E                 # tie rounds to even (448) anyway
    assert fp8.encode_one(500.0) == 0x7E                 # saturate instead of NaN
    assert fp8.encode_one(1e30) == 0x7E
    assert fp8.encode_one(math.inf) == 0x7E
    assert fp8.encode_one(-math.inf) == 0xFE
    assert fp8.encode_one(math.nan) == 0x7F
    assert fp8.encode_one(-0.0) == 0x80


def test_ties_round_to_even():
    # halfway between 1.0 (m=0) and 1.125 (m=1) -> 1.0 ; between 1.125 and 1.25 -> 1.25
    assert fp8.encode_one(1.0625) == 0x38
    assert fp8.encode_one(1.1875) == 0x3A
    # subnormal spacing 2^-9: 1.5 * 2^-9 -> 2 * 2^-9 (even), 0.5 * 2^-9 -> 0
    assert fp8.encode_one(1.5 * 2.0 ** -9) == 0x02
    assert fp8.encode_one(0.5 * 2.0 ** -9) == 0x00
    # top of the subnormals rounds into the first normal
    assert fp8.encode_one(7.5 * 2.0 ** -9) == 0x08


def test_encode_matches_torch_over_all_bf16_at_eight_scales():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = bits.to(torch.float32)
    x = x[torch.isfinite(x)]
    xs = x.numpy()
    for scale in (0.5, 1.0, 1.0 / 3.0, 0.0123, 7.0, 448.0 / 5.1, 2.0 ** -10, 3.3e-3):
        inv = np.float32(1.0) / np.float32(scale)
        with np.errstate(over="ignore"):
            prod = (xs * inv).astype(np.float32)
        keep = np.abs(prod) < 464.0                      # torch's cast does not saturate
        ours = fp8.quantize(xs[keep], inv)
        lib = torch.from_numpy(prod[keep]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(ours, lib), scale
        big = xs[~keep]
        if len(big):
            with np.errstate(over="ignore"):
                q = fp8.quantize(big, inv)
            assert np.all((q == 0x7E) | (q == 0xFE))


def test_dequantize_is_code_times_scale():
    codes = np.arange(256)
    codes = codes[~np.isnan(fp8.decode_table())]
    d = fp8.dequantize(codes, np.float32(0.25))
    assert np.array_equal(d, fp8.decode_table()[codes] * 0.25)


def test_bf16_table_quantize_equals_elementwise():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 65536, size=4000).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    for inv in (np.float32(1.0) / np.float32(0.011), np.float32(3.0)):
        with np.errstate(over="ignore", invalid="ignore"):
            want = fp8.quantize(vals, inv)
        assert np.array_equal(fp8.quantize_bf16_bits(bits, inv), want)
