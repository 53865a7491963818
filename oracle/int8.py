"""Symmetric INT8 absmax quantiser: the comparator and degrade path of the TACO
FP8 operator (CPU).

TEST INFRASTRUCTURE, NOT PRODUCT CODE, like the rest of ``oracle/``.

The pages argue against INT8 for tensor-parallel intermediate tensors
[TACO pt-summary, 1 (TP tensors are dense near zero with a long tail) and 2.A
(INT8's uniform spacing sends many distinct small values to the same integer,
E4M3's exponent keeps them apart)].  They give no INT8 arithmetic.  The
plainest reading, used here and by the library's INT8 path, is exact
arithmetic with a rounding only where a value is stored:

  A      = max |x| over the tensor (per-tensor) or over block k (per-block)
  s      = fp32(127 / A), 1 if A = 0                  (the stored scale)
  code   = clamp(round_half_even(x * s), -127, 127)  (exact product)
  x_hat  = bf16_RNE(code / s)                         (exact quotient)

Blocks are B consecutive elements of a row, as in the FP8 operator.

Why the fp64 steps below are exact (so this is the definition written out,
not an approximation of it):
  * x * s: x is bf16 (at most 8 significant bits) and s is fp32 (at most 24),
    so the product has at most 32 significant bits and fp64 (53) holds it
    exactly; np.rint then rounds half to even.
  * fp32(127 / A) through fp64: A = m 2^e with m odd and m < 2^8.  Unless
    m divides 127 (then the quotient is exact), 127 / A has an infinite
    binary expansion, and in the expansion of r / m (0 < r < m) no run of
    equal bits is longer than 8: a run of k zeros needs a remainder r' with
    r' 2^k < m, a run of k ones (m - r') 2^k < m, both impossible once
    2^k >= m.  Rounding to fp64 first and then to fp32 could differ from one
    rounding only if the fp64 value sat exactly on an fp32 midpoint, which
    needs a run of 28 equal bits.  So the two roundings agree.
  * bf16(code / s) through fp64: let mid be any bf16 midpoint (9 significant
    bits) and s = m 2^f (m odd, m < 2^24).  mid * s is a multiple of the
    lowest bit of mid times that of s and has at most 33 significant bits,
    so code - mid * s is 0 or at least 2^-33 |code| in magnitude: the exact
    quotient is either a midpoint or at least 2^-34 (relative) away from
    every midpoint, far more than fp64's 2^-53 rounding, which therefore
    never moves it onto or across one.  One rounding from fp64 to bf16 gives
    the correctly rounded result.
"""
from __future__ import annotations

import numpy as np

from .taco_oracle import bf16_bits_to_f64, f64_to_bf16_bits

QMAX_INT8 = 127


def int8_scale(absmax: np.ndarray) -> np.ndarray:
    """s = fp32(127 / A), 1 where A = 0."""
    a = np.asarray(absmax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    return np.where(a > 0, QMAX_INT8 / safe, 1.0).astype(np.float32)


def _codes(x64: np.ndarray, s) -> np.ndarray:
    """clamp(round_half_even(x * s)) with the exact product."""
    v = x64 * np.asarray(s, dtype=np.float32).astype(np.float64)
    return np.clip(np.rint(v), -QMAX_INT8, QMAX_INT8).astype(np.int8)


def _x64(x_bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))     # exact


def quantize_int8(x_bits: np.ndarray, s) -> np.ndarray:
    """Codes of x under a given per-tensor scale s (the second half of
    compress_int8_tensor, for tensors whose maximum is known elsewhere)."""
    return _codes(_x64(x_bits), np.float32(s))


def compress_int8_tensor(x_bits: np.ndarray):
    """Per-tensor absmax INT8: (codes int8 [T, H], s float32)."""
    x = _x64(x_bits)
    s = int8_scale(np.max(np.abs(x)) if x.size else 0.0)
    return _codes(x, s), np.float32(s)


def compress_int8_block(x_bits: np.ndarray, block: int):
    """Per-block absmax INT8: (codes int8 [T, H], s float32 [T, H / block])."""
    x = _x64(x_bits)
    T, H = x.shape
    if block < 1 or H % block:
        raise ValueError("hidden must be a multiple of block")
    xb = x.reshape(-1, block)
    s = int8_scale(np.max(np.abs(xb), axis=1))
    q = _codes(xb, s[:, None])
    return q.reshape(T, H), s.reshape(T, H // block)


def _scale_per_element(q: np.ndarray, s, block: int) -> np.ndarray:
    s = np.asarray(s, dtype=np.float32)
    if block == 0:
        return np.full(q.shape, s.reshape(-1)[0], dtype=np.float32)
    T, H = q.shape
    return np.repeat(s.reshape(T, H // block), block, axis=1)


def decompress_int8_f64(q: np.ndarray, s, block: int) -> np.ndarray:
    """code / s in fp64 (see the header: within 2^-53 of exact, never across
    a bf16 rounding boundary); block = 0: one scale per tensor."""
    se = _scale_per_element(q, s, block).astype(np.float64)
    return np.asarray(q, dtype=np.int8).astype(np.float64) / se


def decompress_int8(q: np.ndarray, s, block: int) -> np.ndarray:
    """bf16 bits of code / s, one rounding to nearest even."""
    return f64_to_bf16_bits(decompress_int8_f64(q, s, block))
