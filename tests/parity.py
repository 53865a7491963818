"""Comparison of GPU results with the oracle (test infrastructure).

Bars (written into every parity test):
  * alpha and s: within 1e-6 relative of the oracle's fp32 values;
  * FP8 codes: identical except at most 1e-4 of them, each off by at most one
    code step, where a step is measured on the signed ordinal
    ord(c) = +-(c & 0x7F) (so +0 and -0 are equal);
  * decompressed bf16: within 1e-3 relative Frobenius error of the oracle.
Stricter, from the arithmetic: a GPU result may differ from the oracle only
where the oracle's exact (fp64) value lies within the GPU's fp32 rounding
error of the rounding boundary between the two results.  The fp32 error bound
used is standard: every fp32 add, multiply or fma contributes at most 2^-24
times the magnitude of its result, so a value formed by k roundings from terms
t_i is within k * 2^-24 * sum|t_i| of exact.
"""
from __future__ import annotations

import numpy as np

import oracle

U32 = 2.0 ** -24          # fp32 unit roundoff


def ordinal(codes):
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def value_of_ordinal(o):
    o = np.asarray(o, dtype=np.int64)
    v = oracle.e4m3_decode(np.abs(o).astype(np.uint8))
    return np.where(o < 0, -v, v)


def check_scales(alpha_gpu, s_gpu, alpha_ref, s_ref, rtol=1e-6):
    a_g = np.asarray(alpha_gpu, dtype=np.float64).reshape(-1)
    a_o = np.asarray(alpha_ref, dtype=np.float64).reshape(-1)
    rel_a = np.max(np.abs(a_g - a_o) / a_o) if a_o.size else 0.0
    rel_s = abs(float(s_gpu) - float(s_ref)) / float(s_ref)
    assert rel_a <= rtol, f"alpha relative error {rel_a:.3e} > {rtol}"
    assert rel_s <= rtol, f"scale relative error {rel_s:.3e} > {rtol}"
    return rel_a, rel_s


def _scale_of_blocks(s_ref, blocks):
    """The post-rotation scale of each listed block: s_ref is one per-tensor
    value or an array with one value per block."""
    sv = np.asarray(s_ref, dtype=np.float32).astype(np.float64).reshape(-1)
    return np.full(len(blocks), sv[0]) if sv.size == 1 else sv[blocks]


def check_codes(q_gpu, q_ref, x_bits, alpha_ref, s_ref, block, max_frac=1e-4):
    """FP8 codes: bar plus the near-tie justification of every mismatch.
    Values beyond +-448 saturate on both sides, so they never mismatch."""
    og, oo = ordinal(q_gpu).reshape(-1), ordinal(q_ref).reshape(-1)
    diff = og - oo
    bad = np.nonzero(diff)[0]
    frac = bad.size / max(og.size, 1)
    assert np.all(np.abs(diff) <= 1), f"a code differs by {np.max(np.abs(diff))} steps"
    assert frac <= max_frac, f"{bad.size} codes differ ({frac:.2e} > {max_frac})"
    if bad.size:
        B = block
        blocks = np.unique(bad // B)
        xb = oracle.bf16_bits_to_f64(np.asarray(x_bits).reshape(-1, B)[blocks])
        a = np.asarray(alpha_ref, dtype=np.float32).reshape(-1)[blocks]
        y = oracle.hadamard_rotate(xb, a)                      # exact rotated values
        sb = _scale_of_blocks(s_ref, blocks)
        v = sb[:, None] * y                                    # the value the code encodes
        pos = {b: i for i, b in enumerate(blocks)}
        rows = np.array([pos[b] for b in bad // B])
        cols = bad % B
        vv = v[rows, cols]
        mid = (value_of_ordinal(og[bad]) + value_of_ordinal(oo[bad])) / 2
        # GPU error of s*y: the rotation in fp32 (log2 B + 1 roundings of partial
        # sums bounded by sum|x|), the product alpha*s/sqrt(B)*h (3 roundings), and
        # the 1e-6 relative latitude allowed on alpha and s themselves.
        l1 = np.sum(np.abs(xb), axis=1)[rows]
        k = np.log2(B) + 1
        bound = (sb[rows] * a[rows].astype(np.float64) / np.sqrt(B) * k * U32 * l1
                 + (3 * U32 + 2e-6) * np.abs(vv))
        far = np.abs(vv - mid) > bound
        assert not np.any(far), (
            f"{np.sum(far)} code mismatches are not at a rounding tie, e.g. value {vv[far][0]!r} "
            f"midpoint {mid[far][0]!r}")
    return frac


def bf16_neighbours_ok(got_bits, ref_bits, exact, err_bound, max_frac):
    """bf16 results: equal to the oracle's, or its neighbour where the exact
    value is within err_bound of the rounding boundary between the two."""
    g = oracle.bf16_bits_to_f64(np.asarray(got_bits).reshape(-1))
    r = oracle.bf16_bits_to_f64(np.asarray(ref_bits).reshape(-1))
    ex = np.asarray(exact, dtype=np.float64).reshape(-1)
    eb = np.asarray(err_bound, dtype=np.float64).reshape(-1)
    bad = np.nonzero(g != r)[0]
    frac = bad.size / max(g.size, 1)
    assert frac <= max_frac, f"{bad.size} bf16 outputs differ ({frac:.2e} > {max_frac})"
    if bad.size:
        mid = (g[bad] + r[bad]) / 2
        # both must be adjacent bf16 values straddling the exact value's boundary
        tol = eb[bad] + 4 * U32 * np.abs(ex[bad])
        far = np.abs(ex[bad] - mid) > tol
        assert not np.any(far), (
            f"{np.sum(far)} bf16 mismatches are not at a rounding tie: got {g[bad][far][0]!r} "
            f"want {r[bad][far][0]!r} exact {ex[bad][far][0]!r}")
    return frac


def rel_frobenius(got_bits, ref_bits):
    g = oracle.bf16_bits_to_f64(np.asarray(got_bits))
    r = oracle.bf16_bits_to_f64(np.asarray(ref_bits))
    n = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / n) if n > 0 else float(np.linalg.norm(g))


def decompress_error_bound(q, alpha, s, block):
    """Absolute fp32 error bound of the GPU decompression per element: the
    rotation of decoded codes (log2 B + 1 roundings over sum|dec|) scaled by
    1/(alpha s sqrt B), plus 4 roundings of the scale chain (s per tensor or
    per block)."""
    B = block
    d = np.abs(oracle.e4m3_decode(np.asarray(q)).reshape(-1, B))
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
    sv = _scale_of_blocks(s, np.arange(a.size))
    k = np.log2(B) + 1
    per_block = k * U32 * np.sum(d, axis=1) / (a * sv * np.sqrt(B))
    return np.repeat(per_block, B)


def decompress_sum_error_bound(parts, block):
    """As decompress_error_bound, for the fused sum: each part's weighted
    decoded code is rounded and then added (2 P roundings), then log2 B + 1
    roundings in the rotation."""
    B = block
    P = len(parts)
    tot = None
    for q, alpha, s in parts:
        d = np.abs(oracle.e4m3_decode(np.asarray(q)).reshape(-1, B))
        a = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1)
        w = d / (a[:, None] * np.float64(np.float32(s)))
        tot = w if tot is None else tot + w
    k = 2 * P + np.log2(B) + 2
    per_block = k * U32 * np.sum(tot, axis=1) / np.sqrt(B)
    return np.repeat(per_block, B)
