"""Quantiser comparison and ablation on the synthetic workloads (oracle/ablation.py).

Page-level behaviour, asserted where the pages make a claim and the synthetic
tensors bear it out [TACO pt-summary, 1 and 2.A: uniform INT8 collapses the
dense near-zero values of TP tensors, E4M3 keeps them; 2.B.1: ASH spreads each
block's near-zero cluster over the FP8 range]:
  * per-tensor INT8 rounds nearly all nonzero values to zero, TACO almost none;
  * TACO's reconstruction error is below per-tensor INT8's;
  * ASH lowers the zero collapse of FP8, with and without the rotation.
The full table (also the measurements the pages do not claim anything about)
is printed with -s.  The GPU test checks that the library's own round trip has
the oracle's error and collapse on the same tensors.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import ablation
from fp8_compression_tensor_taco_amd import workloads as W

CASES = [("tiny", 256, 0), ("gpt3_6p7b_act", 64, 0), ("gpt3_6p7b_grad", 64, 1), ("qwen_7b", 32, 0)]


@pytest.fixture(scope="module")
def tab():
    wl = {n: W.bf16_bits(W.make(n, seed=s, tokens=t)) for n, t, s in CASES}
    blk = {n: W.WORKLOADS[n].block for n, _, _ in CASES}
    t = ablation.table(wl, blk)
    for name, row in t.items():
        print(f"\n{name}")
        for m, d in row.items():
            print(f"  {m:13s} rel_err {d['rel_err']:.4f} snr {d['snr_db']:6.2f} dB "
                  f"collapse {d['collapse']:.4f} small_rel_err {d['small_rel_err']:.4f}")
    return t


def test_int8_collapses_the_near_zero_values_taco_does_not(tab):
    for name, row in tab.items():
        assert row["int8_tensor"]["collapse"] >= 0.9, name
        assert row["taco"]["collapse"] <= 1e-3, name
        assert row["taco"]["rel_err"] < row["int8_tensor"]["rel_err"], name


def test_ash_lowers_fp8_zero_collapse(tab):
    for name, row in tab.items():
        assert row["fp8_ash"]["collapse"] < row["fp8_plain"]["collapse"], name
        assert row["taco"]["collapse"] <= row["fp8_hadamard"]["collapse"], name


def test_methods_reduce_to_known_cases():
    """A tensor of one repeated power of two: every method is exact."""
    x = oracle.f64_to_bf16_bits(np.full((2, 256), 0.25))
    for m in ablation.METHODS:
        r, _ = ablation.quantise(m, x, 64)
        assert np.allclose(r, 0.25, rtol=0, atol=1e-12), m
    with pytest.raises(ValueError):
        ablation.quantise("nope", x, 64)


@pytest.mark.gpu
def test_gpu_round_trip_has_the_oracles_error():
    """The library's own round trip (GPU compress, GPU decompress) has the
    oracle's reconstruction error and the oracle's share of zero codes."""
    import fp8_compression_tensor_taco_amd as taco
    for name, tokens, seed in CASES:
        bits = W.bf16_bits(W.make(name, seed=seed, tokens=tokens))
        B = W.WORKLOADS[name].block
        x = oracle.bf16_bits_to_f64(bits)
        q_o, a_o, s_o = oracle.compress(bits, B)
        r_o = oracle.bf16_bits_to_f64(oracle.decompress(q_o, a_o, s_o, B))
        q, a, s = taco.compress(W.from_bits(bits).cuda(), B)
        r_g = oracle.bf16_bits_to_f64(W.bf16_bits(taco.decompress(q, a, s, B)))
        rel_o = np.linalg.norm(r_o - x) / np.linalg.norm(x)
        rel_g = np.linalg.norm(r_g - x) / np.linalg.norm(x)
        assert abs(rel_g - rel_o) <= 1e-2 * rel_o, name
        zeros_o = np.mean(q_o & 0x7F == 0)
        zeros_g = np.mean(q.cpu().numpy() & 0x7F == 0)
        assert abs(zeros_g - zeros_o) <= 1e-4, name


def _kurtosis(v):
    return float(np.mean(v ** 4) / np.mean(v ** 2) ** 2)


def test_rotation_makes_blocks_gaussian_like():
    """The rotation turns each block's heavy-tailed values into a distribution
    close to a Gaussian [TACO pt-summary, 2.B.1]: on every synthetic workload
    the pooled kurtosis of the ASH-scaled blocks is far from 3 (heavy tails)
    and that of the rotated blocks is at least ten times closer.  For iid
    Gaussian blocks the rotation is an orthogonal map, so the rotated values
    stay Gaussian (kurtosis 3 within sampling error)."""
    for name, tokens, seed in CASES:
        B = W.WORKLOADS[name].block
        x = oracle.bf16_bits_to_f64(W.bf16_bits(W.make(name, seed=seed, tokens=tokens))).reshape(-1, B)
        x = x[np.any(x != 0, axis=1)]
        a = oracle.ash_scale(oracle.block_energy(x), 1.0)
        kx = _kurtosis(x * a.astype(np.float64)[:, None])
        ky = _kurtosis(oracle.hadamard_rotate(x, a))
        assert abs(ky - 3) * 10 < abs(kx - 3), (name, kx, ky)
    g = np.random.default_rng(0).standard_normal((4096, 128))
    bits = oracle.f64_to_bf16_bits(g)
    xg = oracle.bf16_bits_to_f64(bits)
    yg = oracle.hadamard_rotate(xg, oracle.ash_scale(oracle.block_energy(xg), 1.0))
    assert abs(_kurtosis(yg) - 3) < 0.05


def test_compressed_volume_is_about_45_percent_smaller():
    """Codes, block scales and the tensor scale against the bf16 tensor: the
    ratio is 1/2 + 2/B (+ 4 bytes), a saving of 47-49% per tensor, in line
    with the average volume reduction the pages report for training
    [TACO zh-news, results section: about 45% less communication volume]."""
    for name, tokens, seed in CASES:
        B = W.WORKLOADS[name].block
        bits = W.bf16_bits(W.make(name, seed=seed, tokens=tokens))
        q, a, s = oracle.compress(bits, B)
        ratio = (q.nbytes + a.nbytes + np.float32(s).nbytes) / bits.nbytes
        assert ratio == pytest.approx(0.5 + 2 / B + 4 / bits.nbytes, rel=0, abs=1e-12)
        assert ratio <= 0.55
