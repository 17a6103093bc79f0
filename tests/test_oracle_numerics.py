"""Pins of the oracle's number formats against torch's own casts (an independent library).

Modelled on the exhaustive codepoint check the patch page "qwen4_exp: FP8 E4M3 KV reader for
QSA" describes for its e4m3 decoder: every code is compared, not a sample.
"""

import numpy as np
import torch

from oracle.numerics import (bf16_bits_to_f64, e4m3_bits_to_f64, f32_to_bf16_bits,
                             f64_to_bf16_bits, f64_to_e4m3_bits)


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_random_and_specials():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * np.float32(5.0),
        rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45, -1e-45, 1.0000001,
                  1.00390625, 1.01171875, 1.0078125], dtype=np.float32),
    ])
    x = x[~np.isnan(x)]
    assert np.array_equal(f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0.
    assert f32_to_bf16_bits(np.float32(1.0 + 2.0 ** -8)) == 0x3F80
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: -> 1 + 2^-6.
    assert f32_to_bf16_bits(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82


def test_bf16_decode_is_exact_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(vals, ref, equal_nan=True)
    finite = np.isfinite(vals)
    assert np.array_equal(f64_to_bf16_bits(vals[finite]), bits[finite])


def test_e4m3_cast_matches_torch_on_every_bf16_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    mine = f64_to_e4m3_bits(vals)
    ref = (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
           .to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    nan_mine = (mine & 0x7F) == 0x7F
    nan_ref = (ref & 0x7F) == 0x7F
    assert np.array_equal(nan_mine, nan_ref)
    assert np.array_equal(mine[~nan_mine], ref[~nan_ref])


def test_e4m3_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint32).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e4m3_bits_to_f64(codes), ref, equal_nan=True)


def test_e4m3_grid_landmarks():
    # OCP e4m3fn: max finite 448, min normal 2^-6, min subnormal 2^-9, NaN at 0x7F / 0xFF.
    assert e4m3_bits_to_f64(np.uint8(0x7E)) == 448.0
    assert e4m3_bits_to_f64(np.uint8(0x08)) == 2.0 ** -6
    assert e4m3_bits_to_f64(np.uint8(0x01)) == 2.0 ** -9
    assert np.isnan(e4m3_bits_to_f64(np.uint8(0x7F)))
    assert np.isnan(e4m3_bits_to_f64(np.uint8(0xFF)))
    # 17 lies halfway between 16 and 18 -> even mantissa -> 16; 19 -> 20.
    assert f64_to_e4m3_bits(np.float64(17.0)) == f64_to_e4m3_bits(np.float64(16.0))
    assert f64_to_e4m3_bits(np.float64(19.0)) == f64_to_e4m3_bits(np.float64(20.0))
