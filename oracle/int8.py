"""Symmetric INT8 absmax quantiser: the comparator and degrade path of the TACO
FP8 operator (CPU).

TEST INFRASTRUCTURE, NOT PRODUCT CODE, like the rest of ``oracle/``.

The pages argue against INT8 for tensor-parallel intermediate tensors
[TACO pt-summary, 1 (TP tensors are dense near zero with a long tail) and 2.A
(INT8's uniform spacing sends many distinct small values to the same integer,
E4M3's exponent keeps them apart)].  They give no INT8 arithmetic; the
plainest reading, used here and by the library's INT8 path:

  A      = max |x| over the tensor (per-tensor) or over block k (per-block)
  s      = fp32(127 / A), 1 if A = 0
  code   = clamp(round_half_even(fp32(x * s)), -127, 127)         (int8)
  x_hat  = bf16_RNE(fp32(code * fp32(1 / s)))

Reading: the product x * s, the reciprocal and the reconstruction are each
rounded to fp32 once, because the quantised code is decided in the
precision the kernel computes in (x is bf16, so fp32(x) is exact); fp64 would
decide a few near-tie codes differently.  numpy's float32 operations are
IEEE single precision with round-to-nearest-even, as the GPU's are.  Blocks
are B consecutive elements of a row, as in the FP8 operator.
"""
from __future__ import annotations

import numpy as np

from .taco_oracle import bf16_bits_to_f64, f64_to_bf16_bits

QMAX_INT8 = 127


def int8_scale(absmax: np.ndarray) -> np.ndarray:
    """s = fp32(127 / A) (fp32 division), 1 where A = 0."""
    a = np.asarray(absmax, dtype=np.float32)
    safe = np.where(a > 0, a, np.float32(1.0))
    return np.where(a > 0, np.float32(QMAX_INT8) / safe, np.float32(1.0)).astype(np.float32)


def _codes(x32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    v = (x32 * s32).astype(np.float32)                     # one fp32 rounding
    return np.clip(np.rint(v), -QMAX_INT8, QMAX_INT8).astype(np.int8)


def _x32(x_bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16)).astype(np.float32)   # exact


def quantize_int8(x_bits: np.ndarray, s) -> np.ndarray:
    """Codes of x under a given per-tensor scale s (the second half of
    compress_int8_tensor, for tensors whose maximum is known elsewhere)."""
    return _codes(_x32(x_bits), np.float32(s))


def compress_int8_tensor(x_bits: np.ndarray):
    """Per-tensor absmax INT8: (codes int8 [T, H], s float32)."""
    x = _x32(x_bits)
    s = int8_scale(np.max(np.abs(x)) if x.size else np.float32(0.0))
    return _codes(x, s), np.float32(s)


def compress_int8_block(x_bits: np.ndarray, block: int):
    """Per-block absmax INT8: (codes int8 [T, H], s float32 [T, H / block])."""
    x = _x32(x_bits)
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


def decompress_int8(q: np.ndarray, s, block: int) -> np.ndarray:
    """bf16 bits of fp32(code * fp32(1 / s)); block = 0: one scale per tensor."""
    se = _scale_per_element(q, s, block)
    r = (np.float32(1.0) / se).astype(np.float32)            # fp32 division
    v = (np.asarray(q, dtype=np.int8).astype(np.float32) * r).astype(np.float32)
    return f64_to_bf16_bits(v.astype(np.float64))


def decompress_int8_f64(q: np.ndarray, s, block: int) -> np.ndarray:
    """code / s in fp64 (no output rounding), for error measurements."""
    se = _scale_per_element(q, s, block).astype(np.float64)
    return np.asarray(q, dtype=np.int8).astype(np.float64) / se
