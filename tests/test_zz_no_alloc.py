"""taco_compress_noalloc: taco_compress with the workspace in the library's own
device scratch, for callers that cannot allocate.  Checked through the C ABI
against taco_compress_ex on the same input, bitwise (the same kernels), on
consecutive calls that share the scratch, the second with a smaller input;
on both pass structures; and repeated, so that every call finds the state the
previous one left.  The outputs of the large call are also held to the
oracle's bars on sampled rows."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_compression_tensor_taco_amd import workloads as W

import parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def taco():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no CPU fallback exists)"
    import fp8_compression_tensor_taco_amd as taco
    taco.load()
    return taco


def outputs(T, H, B):
    return (torch.empty((T, H), dtype=torch.uint8, device="cuda"),
            torch.empty((T, H // B), dtype=torch.float32, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"))


def noalloc(taco, x, B, flags):
    """One taco_compress_noalloc call through the C ABI."""
    T, H = x.shape
    q, a, s = outputs(T, H, B)
    lib = taco.load()
    st = lib.taco_compress_noalloc(ctypes.c_void_p(x.data_ptr()), T, H, B, ctypes.c_float(1.0),
                                   ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                                   ctypes.c_void_p(s.data_ptr()), flags, 0,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.taco_status_string(st).decode()
    return q, a, s


def reference(taco, x, B, flags):
    """The same compression through taco_compress_ex on a workspace of its own."""
    T, H = x.shape
    q, a, s = outputs(T, H, B)
    ws = torch.zeros(taco.workspace_bytes(T, H, B), dtype=torch.uint8, device="cuda")
    lib = taco.load()
    st = lib.taco_compress_ex(ctypes.c_void_p(x.data_ptr()), T, H, B, ctypes.c_float(1.0),
                              ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                              ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                              ws.numel(), flags, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.taco_status_string(st).decode()
    return q, a, s


CASES = [("gpt3_6p7b_act", 4096, 128), ("tiny", 256, 64)]     # the second smaller


@pytest.mark.parametrize("flags", [0, 1])
def test_noalloc_matches_compress_on_consecutive_calls(taco, flags):
    for rep in range(2):
        for name, tokens, B in CASES:
            print(f"[case] noalloc {name} tokens={tokens} block={B} flags={flags} rep={rep}", flush=True)
            x = W.make(name, seed=tokens + rep, tokens=tokens).cuda()
            got = noalloc(taco, x, B, flags)
            ref = reference(taco, x, B, flags)
            torch.cuda.synchronize()
            for g, r in zip(got, ref):
                assert torch.equal(g, r)
            assert not bool(((got[0] & 0x7F) == 0x7F).any())          # no barrier timeout (NaN codes)


def test_noalloc_against_the_oracle(taco):
    """The large call's codes, alpha and s against the oracle on sampled rows
    (s needs the whole tensor, so the oracle runs on all of it)."""
    name, T, B = CASES[0]
    bits = W.bf16_bits(W.make(name, seed=99, tokens=T))
    q, a, s = noalloc(taco, W.from_bits(bits).cuda(), B, 0)
    torch.cuda.synchronize()
    q_o, a_o, s_o = oracle.compress(bits, B)
    parity.check_scales(a.cpu().numpy(), float(s.item()), a_o, s_o)
    rows = [0, 1, 2047, 4095]
    parity.check_codes(q.cpu().numpy()[rows], q_o[rows], bits[rows], a_o[rows], s_o, B)


def test_noalloc_rejects_bad_arguments(taco):
    lib = taco.load()
    f = ctypes.c_float(1.0)
    assert lib.taco_compress_noalloc(None, 8, 128, 64, f, None, None, None, 0, 0, None) == 1
    x = torch.empty((8, 128), dtype=torch.bfloat16, device="cuda")
    q, a, s = outputs(8, 128, 64)
    p = [ctypes.c_void_p(t.data_ptr()) for t in (x, q, a, s)]
    assert lib.taco_compress_noalloc(p[0], 8, 96, 64, f, p[1], p[2], p[3], 0, 0, None) == 3
    assert lib.taco_compress_noalloc(p[0], 8, 128, 64, f, p[1], p[2], p[3], 4, 0, None) == 9   # unknown flag
    assert lib.taco_compress_noalloc(p[0], 8, 128, 64, f, p[0], p[2], p[3], 0, 0, None) == 10  # q is x
