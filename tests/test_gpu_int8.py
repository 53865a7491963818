"""GPU parity of the INT8 degrade path (taco_compress_int8 / taco_decompress_int8,
through the C ABI) against oracle/int8.py.

Integer and byte work, so the bar is bit-exact: codes, scales and the bf16
reconstruction equal the oracle's on the same seeded input (both sides take
every rounding decision in fp32).  Cases: small shapes with ragged tails
(fewer pieces than one wavefront, partial workgroups, several trips of the
grid-stride loops), every block size and the per-tensor scale, the workloads
at full size, zero tensors and blocks, ties, extreme magnitudes, and a
workspace shared with the FP8 compress.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_compression_tensor_taco_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def taco():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no CPU fallback exists)"
    import fp8_compression_tensor_taco_amd as taco
    taco.load()
    return taco


def run_int8(taco, bits, block):
    T, H = bits.shape
    print(f"[case] int8 shape=({T},{H}) block={block}", flush=True)
    if block == 0:
        q_o, s_o = oracle.compress_int8_tensor(bits)
    else:
        q_o, s_o = oracle.compress_int8_block(bits, block)
    y_o = oracle.decompress_int8(q_o, s_o, block)
    q, s = taco.compress_int8(W.from_bits(bits).cuda(), block)
    y = taco.decompress_int8(q, s, block)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_o)
    s_g = s.cpu().numpy().reshape(-1)
    assert np.array_equal(s_g.view(np.uint32), np.asarray(s_o, dtype=np.float32).reshape(-1).view(np.uint32))
    assert np.array_equal(W.bf16_bits(y), y_o)
    # the GPU decompress of the oracle's codes too (no GPU value feeds the check)
    y2 = taco.decompress_int8(torch.from_numpy(q_o).cuda(),
                              torch.from_numpy(np.asarray(s_o, dtype=np.float32).reshape(s.shape)).cuda(), block)
    assert np.array_equal(W.bf16_bits(y2), y_o)


SHAPES = [(1, 8), (3, 24), (1, 256), (5, 768), (131, 512), (64, 1024), (257, 3584)]


@pytest.mark.parametrize("block", [0, 64, 128, 256])
@pytest.mark.parametrize("tokens,hidden", SHAPES)
def test_small_shapes(taco, block, tokens, hidden):
    if block and hidden % block:
        pytest.skip("hidden is not a multiple of the block")
    name = "tiny" if tokens <= 256 and hidden <= 1024 else "qwen_7b"
    bits = W.bf16_bits(W.make(name, seed=tokens + hidden, tokens=tokens))
    run_int8(taco, np.ascontiguousarray(bits[:, :hidden]), block)


@pytest.mark.parametrize("name", ["gpt3_6p7b_act", "gpt3_6p7b_grad", "qwen_7b", "gpt2_1p5b"])
@pytest.mark.parametrize("block", [0, 64, 128])
def test_full_size(taco, name, block):
    wl = W.WORKLOADS[name]
    if block and wl.hidden % block:
        pytest.skip("hidden is not a multiple of the block")
    run_int8(taco, W.bf16_bits(W.make(name, seed=2)), block)


def test_zero_tensor_and_zero_blocks(taco):
    run_int8(taco, np.zeros((4, 512), dtype=np.uint16), 0)
    run_int8(taco, np.zeros((4, 512), dtype=np.uint16), 128)
    x = np.concatenate([np.zeros((2, 128)), np.full((2, 128), -0.375)], axis=1)
    x[1, 0] = -0.0
    run_int8(taco, oracle.f64_to_bf16_bits(x), 128)


def test_ties_and_extreme_magnitudes(taco):
    ties = np.tile(np.array([127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.5, -126.5]), (3, 32))
    run_int8(taco, oracle.f64_to_bf16_bits(ties), 0)
    run_int8(taco, oracle.f64_to_bf16_bits(ties), 64)
    base = oracle.bf16_bits_to_f64(W.bf16_bits(W.make("tiny", seed=11, tokens=8)))
    for e in (-60, -30, 30, 60):
        run_int8(taco, oracle.f64_to_bf16_bits(base * 2.0 ** e), 0)
        run_int8(taco, oracle.f64_to_bf16_bits(base * 2.0 ** e), 256)


def test_workspace_shared_with_fp8_compress(taco):
    """The per-tensor INT8 call uses only the partial-maximum region of a
    compress workspace: fused FP8 compresses on the same workspace stay
    bitwise equal to those on a fresh one, and no barrier times out."""
    x = W.make("gpt3_6p7b_act", seed=5).cuda()
    ws = torch.zeros(taco.workspace_bytes(4096, 4096, 128), dtype=torch.uint8, device="cuda")
    ref = [t.clone() for t in taco.compress(x, 128, workspace=torch.zeros_like(ws))]
    for _ in range(3):
        q8, s8 = taco.compress_int8(x, 0, workspace=ws)
        got = taco.compress(x, 128, workspace=ws)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    assert not taco.workspace_timed_out(ws)
    q_o, s_o = oracle.compress_int8_tensor(W.bf16_bits(x.cpu()))
    assert np.array_equal(q8.cpu().numpy(), q_o)
