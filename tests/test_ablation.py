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
