"""Pins for the oracle's E4M3FN and bf16 codecs (CPU only).

The E4M3 format is named by the pages [TACO pt-summary, 2.A] and its largest
value Q_max by [TACO pt-summary, 2.B.2]; bit layouts are the OCP OFP8 and bfloat16
definitions.  Pins: hand-derived anchor values, an exhaustive comparison with
torch's own float8_e4m3fn / bfloat16 conversions (an independent library
routine), and structural properties (round trip, monotonicity, ties to even,
saturation).
"""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# --------------------------------------------------------------------- E4M3
def test_e4m3_anchor_values():
    t = oracle.e4m3_table()
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9            # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert t[0x08] == 2.0 ** -6            # smallest normal
    assert t[0x38] == 1.0                  # exponent field 7 = bias
    assert t[0x3F] == 1.875
    assert t[0x40] == 2.0
    assert t[0x7E] == 448.0                # Q_max
    assert t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2        # no infinities, only two NaNs
    assert oracle.Q_MAX == 448.0


def test_e4m3_table_matches_torch_exhaustively():
    ours, ref = oracle.e4m3_table(), torch_e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3_roundtrip_and_monotonic():
    t = oracle.e4m3_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(t[codes]), codes)
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3_ties_go_to_even_code():
    t = oracle.e4m3_table()
    for c in range(0x7E):
        lo, hi = t[c], t[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == even, hex(c)
        assert oracle.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)
        eps = (hi - lo) * 1e-6
        assert oracle.e4m3_encode(np.array([mid - eps]))[0] == c
        assert oracle.e4m3_encode(np.array([mid + eps]))[0] == c + 1
    # explicit cases worked by hand
    cases = {2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 1.0625: 0x38, 1.1875: 0x3A,
             464.0: 0x7E, 89.6: 0x6B, 179.2: 0x73}
    for v, c in cases.items():
        assert oracle.e4m3_encode(np.array([v]))[0] == c, v


def test_e4m3_saturates_and_keeps_sign_of_zero():
    big = np.array([448.0, 448.5, 463.99, 464.0, 480.0, 1e6, 1e300])
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    assert oracle.e4m3_encode(np.array([0.0]))[0] == 0x00
    assert oracle.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert oracle.e4m3_encode(np.array([-1e-9]))[0] == 0x80
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([np.nan]))


def test_e4m3_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(1234)
    # fp32 values spread over every binade of the format, both signs, plus
    # every exact midpoint (torch rounds fp32 -> e4m3 once, to nearest even)
    mags = np.exp2(rng.uniform(-13, np.log2(448.0), 200_000))
    v = (mags * rng.choice([-1.0, 1.0], mags.size)).astype(np.float32)
    t = oracle.e4m3_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------- bf16
def all_finite_bf16_bits():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f64(b)
    return b[np.isfinite(f)]


def test_bf16_widening_matches_torch_exhaustively():
    b = all_finite_bf16_bits()
    ours = oracle.bf16_bits_to_f64(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_bf16_narrowing_exhaustive_midpoints():
    b = all_finite_bf16_bits()
    assert np.array_equal(oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(b)), b)
    # positive finite patterns in increasing order: 0x0000 .. 0x7F7F
    pos = np.arange(0x0000, 0x7F80, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_bits_to_f64(pos)
    mid = (v[:-1] + v[1:]) / 2                        # exact in fp64
    even = np.where(pos[:-1] % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(oracle.f64_to_bf16_bits(mid), even)
    assert np.array_equal(oracle.f64_to_bf16_bits(-mid), even | 0x8000)
    gap = v[1:] - v[:-1]
    assert np.array_equal(oracle.f64_to_bf16_bits(mid - gap / 8), pos[:-1])
    assert np.array_equal(oracle.f64_to_bf16_bits(mid + gap / 8), pos[1:])
    # past the largest finite value by more than half a step -> infinity
    assert oracle.f64_to_bf16_bits(np.array([3.5e38]))[0] == 0x7F80


def test_bf16_narrowing_matches_torch_on_random_fp32():
    rng = np.random.default_rng(99)
    bits = rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(v.astype(np.float64)), ref)
