"""Quantiser comparison and ablation for the TACO operator (fp64, CPU).

TEST INFRASTRUCTURE, NOT PRODUCT CODE, like the rest of ``oracle/``.

The pages' central numerical argument [TACO pt-summary, 1 (TP tensors are
dense near zero with a long tail) and 2.A (uniform INT8 spacing maps distinct
small values onto the same integer; E4M3's exponent keeps them apart)], and
the roles of the two transforms [2.B.1: ASH spreads each block's near-zero
cluster over the FP8 range, the Hadamard rotation makes the values
Gaussian-like], measured on tensors directly instead of through training:

  int8_tensor    symmetric INT8, one absmax scale per tensor
  int8_block     symmetric INT8, one absmax scale per block
  fp8_plain      E4M3 with one per-tensor scale, no ASH, no rotation
  fp8_hadamard   rotation only (no ASH), per-tensor scale
  fp8_ash        ASH only (no rotation), per-tensor scale
  taco           ASH + rotation + per-tensor scale (oracle.compress)

Readings: the INT8 rows are oracle/int8.py's quantiser (round half to even,
clip at +-127, exact products; the pages give no INT8 details); each FP8
ablation keeps the rest of the method unchanged.
Every function returns the fp64 reconstruction (before any bf16 rounding) and
the values handed to the rounding step, so that collapse can be measured in
the code domain.
"""
from __future__ import annotations

import numpy as np

from . import int8 as i8
from . import taco_oracle as o

METHODS = ("int8_tensor", "int8_block", "fp8_plain", "fp8_hadamard", "fp8_ash", "taco")


def _fp8(v: np.ndarray, s) -> tuple[np.ndarray, np.ndarray]:
    codes = o.e4m3_encode(np.float64(s) * v)
    return o.e4m3_decode(codes) / np.float64(s), np.float64(s) * v


def _tensor_scale(v: np.ndarray, qmax: float) -> np.float32:
    m = float(np.max(np.abs(v))) if v.size else 0.0
    return np.float32(qmax / m) if m > 0 else np.float32(1.0)


def quantise(method: str, x_bits: np.ndarray, block: int, target_energy: float = 1.0):
    """Reconstruction (fp64, shape of x) and the pre-rounding values of one method."""
    x = o.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    T, H = x.shape
    xb = x.reshape(-1, block)
    if method == "int8_tensor":
        q, sc = i8.compress_int8_tensor(x_bits)
        r = i8.decompress_int8_f64(q, sc, 0)
        v = x * np.float64(sc)                       # exact (8- by 24-bit product)
    elif method == "int8_block":
        q, sc = i8.compress_int8_block(x_bits, block)
        r = i8.decompress_int8_f64(q, sc, block)
        v = x * np.repeat(sc, block, axis=1).astype(np.float64)
    elif method == "fp8_plain":
        r, v = _fp8(xb, _tensor_scale(xb, o.Q_MAX))
    elif method == "fp8_hadamard":
        y = xb @ o.hadamard(block).T / np.sqrt(block)
        yr, v = _fp8(y, _tensor_scale(y, o.Q_MAX))
        r = yr @ o.hadamard(block).T / np.sqrt(block)          # H / sqrt(B) is its own inverse
    elif method == "fp8_ash":
        a = o.ash_scale(o.block_energy(xb), target_energy).astype(np.float64)[:, None]
        y = a * xb
        yr, v = _fp8(y, _tensor_scale(y, o.Q_MAX))
        r = yr / a
    elif method == "taco":
        q, alpha, s = o.compress(x_bits, block, target_energy)
        r = o.decompress_f64(q, alpha, s, block).reshape(-1, block)
        y = o.hadamard_rotate(xb, alpha.reshape(-1))
        v = np.float64(s) * y
    else:
        raise ValueError(f"unknown method {method!r}")
    return r.reshape(T, H), v.reshape(T, H)


def metrics(method: str, x_bits: np.ndarray, block: int, target_energy: float = 1.0) -> dict:
    """Error of one method on one tensor:
      rel_err        ||xhat - x|| / ||x||
      snr_db         10 log10(||x||^2 / ||xhat - x||^2)
      collapse       fraction of nonzero values handed to the rounding step
                     that round to zero (the pages' zero collapse)
      small_rel_err  ||xhat - x|| / ||x|| over the elements with |x| at or
                     below the median |x| (the dense region near zero)
    """
    x = o.bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    r, v = quantise(method, x_bits, block, target_energy)
    err = r - x
    nx = np.linalg.norm(x)
    ne = np.linalg.norm(err)
    if method.startswith("int8"):
        zero = np.rint(v) == 0
    else:
        zero = o.e4m3_decode(o.e4m3_encode(v)) == 0
    nonzero = v != 0
    small = np.abs(x) <= np.median(np.abs(x))
    ns = np.linalg.norm(x[small])
    return {
        "rel_err": float(ne / nx) if nx > 0 else 0.0,
        "snr_db": float(10 * np.log10(nx ** 2 / ne ** 2)) if ne > 0 else float("inf"),
        "collapse": float(np.mean(zero[nonzero])) if nonzero.any() else 0.0,
        "small_rel_err": float(np.linalg.norm(err[small]) / ns) if ns > 0 else 0.0,
    }


def table(workloads: dict, block_of: dict, target_energy: float = 1.0) -> dict:
    """metrics for every method on every named tensor: {name: {method: dict}}."""
    return {name: {m: metrics(m, bits, block_of[name], target_energy) for m in METHODS}
            for name, bits in workloads.items()}
