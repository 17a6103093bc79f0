"""Number formats used by the oracle: bf16 and OCP e4m3fn, written from their definitions.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this module; only the
tests, the smoke check and the CPU-baseline leg of the benchmark use it.

Values are carried as float64 arrays holding exactly-representable numbers; bit patterns
are carried as uint16 (bf16) or uint8 (e4m3fn) arrays.

Sources
-------
* The indexer keeps its Q and compressed keys either in bf16 or in ``torch.float8_e4m3fn``
  "without scales" (page "vllm.models.qwen4_exp.nvidia.qsa", class ``QSAIndexer``,
  ``__init__``: the ``indexer_kv_dtype`` branch).  e4m3fn is the OCP 8-bit float with 4
  exponent bits (bias 7), 3 mantissa bits, no infinities, and the all-ones magnitude
  0x7F as NaN (the patch page "qwen4_exp: FP8 E4M3 KV reader for QSA", comment of
  ``_decode_e4m3_to_bf16``, names 0x7F/0xFF as the NaN codes).
* Reading taken where the pages are silent: the cast from a wider float to e4m3fn rounds
  to nearest, ties to even, and a magnitude that rounds past 448 becomes NaN -- the
  behaviour of ``Tensor.to(torch.float8_e4m3fn)``, which the unfused Q path calls
  (``q.to(self.indexer_dtype)`` in ``QSAIndexer.forward``).  The tests pin this function
  against torch on every bf16 bit pattern.
"""

from __future__ import annotations

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)


# ----------------------------------------------------------------------------- bf16


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact: bf16 is the top half of a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN -> 0x7FC0."""
    x32 = np.asarray(x32, dtype=np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(np.isnan(x32), np.uint64(BF16_QNAN), r)
    return r.astype(np.uint16)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE).

    The two-step rounding is the canonical chain of this project: the reference computes
    its norms and rotations in float32 and stores bf16 tensors, so every bf16 value the
    oracle produces passes through float32 first.
    """
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (through float32), returned as float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


# ----------------------------------------------------------------------------- e4m3fn


def e4m3_bits_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes -> float64.  exponent field 0 is subnormal (m * 2^-9);
    otherwise (1 + m/8) * 2^(e-7); magnitude 0x7F is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def f64_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float64 (already a float32 value) -> e4m3fn code, round to nearest, ties to even.

    Rounding is done on the grid of e4m3fn values extended by the would-be value of code
    0x7F (480): a result of 480 or beyond, and any NaN input, gives the NaN code.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        # Below the smallest normal (2^-6) the grid step is 2^-9.
        q_sub = np.rint(a * 2.0 ** 9)  # 0..8; 8 is the code of 2^-6
        # Normals: a = f * 2^E with f in [1, 2); the grid step is 2^(E-3).
        _, e = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
        E = e.astype(np.int64) - 1
        q = np.rint(a * np.exp2(3.0 - E))  # 8..16
        carry = q >= 16
        E = np.where(carry, E + 1, E)
        q = np.where(carry, 8, q)
        normal = (E + 7) * 8 + (q - 8)
        code = np.where(a < 2.0 ** -6, q_sub, normal)
        bad = ~np.isfinite(a) | ((a >= 2.0 ** -6) & (E + 7 > 15)) | (code >= 0x7F)
        code = np.where(bad, 0x7F, code).astype(np.int64)
    return (code | sign).astype(np.uint8)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest e4m3fn value (as float64)."""
    return e4m3_bits_to_f64(f64_to_e4m3_bits(x))
