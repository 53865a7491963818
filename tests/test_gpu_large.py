"""Maximum sizes: a [509000, 4224] bf16 tensor (2.15e9 elements, past 2^31, so
every element, block and tile index needs 64 bits; 33 blocks of 128 per row,
so tiles straddle rows and the last one is ragged).

Every expected value comes from the oracle alone:
  * the per-tensor scale: the whole input is copied to the host and streamed
    through the oracle's steps (block energy, ASH scale, rotation) in row
    chunks, keeping a running max|y|; s = fp32(448 / max) is the oracle's
    ds_scale of that max, and the GPU's s must match it to 1e-6;
  * sampled rows (the first, the middle, those around element 2^31, the
    last): codes and alpha against the oracle's under the oracle's s, with the
    bars of the smaller parity tests;
  * decompress and decompress-sum: the sampled rows of the GPU's buffers are
    overwritten with the oracle's codes and alpha, and the scale with the
    oracle's s, before the GPU call, so the checked outputs are the GPU's
    reconstruction of the oracle's compressed rows;
  * INT8: the tensor's max |x| from the host copy.
The input is drawn on the GPU by torch's seeded generator (not by this
library); the host copy of it is the oracle's input.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from fp8_compression_tensor_taco_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu

T, H, B = 509000, 4224, 128
ROWS = [0, 1, T // 2, (1 << 31) // H - 1, (1 << 31) // H, (1 << 31) // H + 1, T - 2, T - 1]
CHUNK = 4096                    # rows per oracle chunk on the host


def _oracle_chunk_max(bits):
    """max |y| of a row chunk: the oracle's steps, in the oracle's order."""
    xb = oracle.bf16_bits_to_f64(bits).reshape(-1, B)
    a = oracle.ash_scale(oracle.block_energy(xb), 1.0)
    return float(np.max(np.abs(oracle.hadamard_rotate(xb, a))))


@pytest.fixture(scope="module")
def big():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no CPU fallback exists)"
    import fp8_compression_tensor_taco_amd as taco
    taco.load()
    assert T * H > (1 << 31)
    print(f"[case] large tensor [{T}, {H}] = {T * H} elements", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(1234)
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    chunk = 32768
    for r in range(0, T, chunk):
        n = min(chunk, T - r)
        v = torch.randn((n, H), generator=gen, device="cuda", dtype=torch.float32)
        v[:, ::211] *= 20.0                                  # outlier columns
        x[r:r + n] = v.to(torch.bfloat16)
    torch.cuda.synchronize()
    print("[case] large tensor: host copy and oracle max", flush=True)
    host = W.bf16_bits(x.cpu())                              # uint16 [T, H], 4.3 GB
    with ThreadPoolExecutor(max_workers=8) as pool:
        amax = max(pool.map(lambda r: _oracle_chunk_max(host[r:r + CHUNK]), range(0, T, CHUNK)))
    s_o = np.float32(oracle.Q_MAX / amax)
    yield taco, x, host, s_o
    del x, host
    torch.cuda.empty_cache()


def rows_bits(t, rows):
    return np.stack([W.bf16_bits(t[r:r + 1].cpu())[0] for r in rows])


def test_large_compress_decompress(big):
    taco, x, host, s_o = big
    q, a, s = taco.compress(x, B)
    torch.cuda.synchronize()
    s_g = np.float32(s.item())
    print(f"[case] large compress: scale {s_g!r} against the oracle's {s_o!r}", flush=True)
    parity.check_scales(np.ones(1), s_g, np.ones(1), s_o)
    assert int(((q & 0x7F) == 0x7F).sum().item()) == 0               # no NaN code
    print("[case] large compress: sampled rows", flush=True)
    xr = host[ROWS]
    xb = oracle.bf16_bits_to_f64(xr).reshape(-1, B)
    a_o = oracle.ash_scale(oracle.block_energy(xb), 1.0)
    a_g = np.stack([a[r].cpu().numpy() for r in ROWS]).reshape(-1)
    parity.check_scales(a_g, s_o, a_o, s_o)
    q_o = oracle.quantize(oracle.hadamard_rotate(xb, a_o), s_o).reshape(len(ROWS), H)
    q_g = np.stack([q[r].cpu().numpy() for r in ROWS])
    a_rows = a_o.reshape(len(ROWS), -1)
    parity.check_codes(q_g, q_o, xr, a_rows, s_o, B)
    # the oracle's compressed rows and scale into the GPU's buffers
    for i, r in enumerate(ROWS):
        q[r] = torch.from_numpy(q_o[i]).cuda()
        a[r] = torch.from_numpy(a_rows[i]).cuda()
    s.fill_(float(s_o))
    print("[case] large decompress: sampled rows", flush=True)
    out = taco.decompress(q, a, s, B)
    torch.cuda.synchronize()
    got = rows_bits(out, ROWS)
    ref = oracle.decompress(q_o, a_rows, s_o, B)
    exact = oracle.decompress_f64(q_o, a_rows, s_o, B)
    parity.bf16_neighbours_ok(got, ref, exact, parity.decompress_error_bound(q_o, a_rows, s_o, B), 0.05)
    assert parity.rel_frobenius(got, ref) <= 1e-3
    del out
    print("[case] large decompress_sum, 2 parts: sampled rows", flush=True)
    out = taco.decompress_sum([(q, a, s), (q, a, s)], B)
    torch.cuda.synchronize()
    got = rows_bits(out, ROWS)
    parts = [(q_o, a_rows, s_o)] * 2
    ref = oracle.decompress_sum(parts, B)
    exact = 2 * oracle.decompress_f64(q_o, a_rows, s_o, B)
    parity.bf16_neighbours_ok(got, ref, exact, parity.decompress_sum_error_bound(parts, B), 0.05)
    assert parity.rel_frobenius(got, ref) <= 1e-3
    del out, q, a, s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("block", [0, B])
def test_large_int8(big, block):
    taco, x, host, _ = big
    print(f"[case] large int8 block={block}", flush=True)
    q, s = taco.compress_int8(x, block)
    torch.cuda.synchronize()
    xr = host[ROWS]
    if block == 0:
        amax = float(oracle.bf16_bits_to_f64(np.max(host & np.uint16(0x7FFF))))   # max |x|, exact
        s_o = oracle.int8_scale(amax)
        assert s.cpu().numpy().view(np.uint32)[0] == np.float32(s_o).view(np.uint32)
        q_o = oracle.quantize_int8(xr, s_o)
        s_cmp = np.float32(s_o)
    else:
        q_o, s_cmp = oracle.compress_int8_block(xr, block)
        s_g = np.stack([s[r].cpu().numpy() for r in ROWS])
        assert np.array_equal(s_g.view(np.uint32), s_cmp.view(np.uint32))
    q_g = np.stack([q[r].cpu().numpy() for r in ROWS])
    assert np.array_equal(q_g, q_o)
    # the decompression of the sampled rows reads exactly the oracle's codes
    # and scales (equal bitwise, asserted above)
    out = taco.decompress_int8(q, s, block)
    torch.cuda.synchronize()
    assert np.array_equal(rows_bits(out, ROWS), oracle.decompress_int8(q_o, s_cmp, block))
    del q, s, out
    torch.cuda.empty_cache()
