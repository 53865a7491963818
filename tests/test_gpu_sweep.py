"""GPU parity on a seeded sweep of small random configurations.

Each case draws a shape (1-200 rows, hidden a multiple of the block up to
4096), a block size, a target energy and an input recipe (activation or
gradient mix, outlier columns, per-row magnitudes) from one seeded generator,
then holds the library to the same element-wise bars against the oracle as
the fixed cases in test_gpu_parity.py: compress and decompress on both pass
structures, a 3-part decompress-sum, and the fused decompress-sum-compress.
"""
import numpy as np
import pytest

import oracle
from fp8_compression_tensor_taco_amd import workloads as W
from test_gpu_parity import Mode, run_decompress_sum, run_decompress_sum_compress, run_round_trip

pytestmark = pytest.mark.gpu

N_CASES = 16


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    block = int(rng.choice([64, 128, 256]))
    tokens = int(rng.integers(1, 201))
    hidden = block * int(rng.integers(1, 4096 // block + 1))
    E = float(2.0 ** rng.uniform(-6, 6))
    mix = str(rng.choice(["act", "grad"]))
    outliers = float(rng.choice([0.0, 20.0, 50.0]))
    rows = bool(rng.integers(0, 2))
    seed = int(rng.integers(0, 2 ** 31))
    return block, tokens, hidden, E, mix, outliers, rows, seed


def bits_of(tokens, hidden, mix, outliers, rows, seed):
    x = W.draw_f64(tokens, hidden, mix, outliers, rows, seed)
    return oracle.f64_to_bf16_bits(x.astype(np.float32).astype(np.float64))


@pytest.fixture(scope="module")
def taco():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU (no CPU fallback exists)"
    import fp8_compression_tensor_taco_amd as taco
    taco.load()
    return taco


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep(taco, case):
    block, tokens, hidden, E, mix, outliers, rows, seed = draw_case(case)
    print(f"[case] sweep {case}: [{tokens}, {hidden}] block {block} E {E:.4g} {mix} "
          f"outliers x{outliers:g} row magnitudes {rows} seed {seed}", flush=True)
    bits = bits_of(tokens, hidden, mix, outliers, rows, seed)
    for path in ("fused", "two_pass"):
        run_round_trip(Mode(taco, path), bits, block, E)
    parts = [bits_of(tokens, hidden, mix, outliers, rows, seed + p) for p in range(3)]
    run_decompress_sum(taco, parts, block)
    run_decompress_sum_compress(taco, parts, block, E)
