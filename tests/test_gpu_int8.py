"""GPU parity of the INT8 degrade path (taco_compress_int8 / taco_decompress_int8,
through the C ABI) against oracle/int8.py.

Integer and byte work, so the bar is bit-exact: codes, scales and the bf16
reconstruction equal the oracle's on the same seeded input.  The oracle
decides every rounding on the exact product x * s and the exact quotient
code / s; the kernels decide them exactly too (an fma residual), and the
adversarial cases below hold products that fp32 rounds onto a half-integer
and quotients that an fp32 reciprocal or division rounds across a bf16
midpoint.  Cases: small shapes with ragged tails
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


@pytest.mark.parametrize("tokens,hidden,block", [(t, h, b) for t, h in SHAPES for b in (0, 64, 128, 256)
                                                 if b == 0 or h % b == 0])
def test_small_shapes(taco, block, tokens, hidden):
    name = "tiny" if tokens <= 256 and hidden <= 1024 else "qwen_7b"
    bits = W.bf16_bits(W.make(name, seed=tokens + hidden, tokens=tokens))
    run_int8(taco, np.ascontiguousarray(bits[:, :hidden]), block)


@pytest.mark.parametrize("name,block", [(n, b) for n in ("gpt3_6p7b_act", "gpt3_6p7b_grad", "qwen_7b", "gpt2_1p5b")
                                        for b in (0, 64, 128) if b == 0 or W.WORKLOADS[n].hidden % b == 0])
def test_full_size(taco, name, block):
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


def _half_way_values(A):
    """bf16 values x <= A whose fp32 product with s = fp32(127 / A) lands
    exactly on a half-integer while the exact product does not (found by
    search over every bf16 value up to A)."""
    v = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    v = v[v <= A]
    s = np.float32(127.0 / np.float64(A))
    p32 = (v * s).astype(np.float32).astype(np.float64)
    exact = v.astype(np.float64) * np.float64(s)
    return v[(p32 - np.floor(p32) == 0.5) & (exact != p32)]


def test_half_way_products(taco):
    """Blocks whose values include A/2 and every other bf16 value whose fp32
    product with s sits exactly half-way while the exact one does not: the
    codes follow the exact product (per block and per tensor)."""
    rng = np.random.default_rng(17)
    cands = (np.arange(0x3C00, 0x4400, dtype=np.uint32) << 16).view(np.float32)   # bf16 in [2^-7, 2^8)
    rows, n = [], 0
    for A in rng.choice(cands, 400, replace=False):
        hw = _half_way_values(A)
        if hw.size == 0:
            continue
        n += hw.size
        row = np.zeros(256)
        row[0] = A
        k = min(hw.size, 127)
        row[1:1 + k] = hw[:k]
        row[128:128 + k] = -hw[:k]
        row[128 + 127] = -A
        rows.append(row)
    assert n >= 100
    bits = oracle.f64_to_bf16_bits(np.array(rows))
    print(f"[case] int8 half-way products: {len(rows)} rows, {n} half-way values", flush=True)
    run_int8(taco, bits, 128)
    run_int8(taco, bits[:1], 0)


def test_decode_quotients_near_bf16_midpoints(taco):
    """Pairs (code, s) where an fp32 reciprocal product or an fp32 division
    rounds to another bf16 value than the exact quotient (found by search),
    decoded per block of 64 on the GPU against the oracle."""
    rng = np.random.default_rng(5)
    s = (rng.uniform(0.5, 2.0, 60000) * 2.0 ** rng.integers(-20, 20, 60000)).astype(np.float32)
    c = np.arange(-127, 128, dtype=np.float32)
    r = (np.float32(1.0) / s).astype(np.float32)
    ref = oracle.f64_to_bf16_bits(c[None, :].astype(np.float64) / s[:, None].astype(np.float64))
    alt1 = oracle.f64_to_bf16_bits((c[None, :] * r[:, None]).astype(np.float32).astype(np.float64))
    alt2 = oracle.f64_to_bf16_bits((c[None, :] / s[:, None]).astype(np.float32).astype(np.float64))
    hard = np.argwhere((alt1 != ref) | (alt2 != ref))
    assert len(hard) >= 10
    q = np.zeros((len(hard), 64), dtype=np.int8)
    q[:, 0] = c[hard[:, 1]].astype(np.int8)
    q[:, 1:] = rng.integers(-127, 128, (len(hard), 63))
    sb = s[hard[:, 0]].reshape(-1, 1)
    print(f"[case] int8 decode near bf16 midpoints: {len(hard)} pairs", flush=True)
    want = oracle.decompress_int8(q, sb, 64)
    got = taco.decompress_int8(torch.from_numpy(q).cuda(), torch.from_numpy(sb).cuda(), 64)
    assert np.array_equal(W.bf16_bits(got), want)
    for i in range(min(len(hard), 8)):                  # one scale per tensor too
        want1 = oracle.decompress_int8(q[i:i + 1], sb[i, 0], 0)
        got1 = taco.decompress_int8(torch.from_numpy(q[i:i + 1]).cuda(),
                                    torch.from_numpy(sb[i]).cuda(), 0)
        assert np.array_equal(W.bf16_bits(got1), want1)
