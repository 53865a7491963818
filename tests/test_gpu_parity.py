"""GPU parity: libtaco (through its C ABI, via the ctypes binding) against the oracle.

Every case runs the GPU kernels and the fp64 oracle on the same seeded bf16
input and compares element by element (see tests/parity.py for the bars):
  * small sizes that span several workgroup tiles and end in a ragged tail;
  * the full workload sizes, in the launch configuration bench.py times;
  * edge cases: zero tensors and blocks, one-hot and constant blocks, a single
    row, extreme magnitudes, negative zeros, every FP8 code.
Inputs for decompress and decompress-sum are the oracle's own compressed
triples, so no oracle input ever comes from the GPU path.
"""
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


def to_gpu_bits(bits):
    return W.from_bits(bits).cuda()


def gpu_triple_np(q, a, s):
    torch.cuda.synchronize()
    return q.cpu().numpy(), a.cpu().numpy(), np.float32(s.cpu().numpy()[0])


# bf16 outputs: every element that differs from the oracle's must be justified by
# the fp32 error bound at a bf16 rounding tie (tests/parity.py); where a block
# mixes a heavy tail with near-zero values the fp32 rotation cancels and that
# bound is wide, so the fraction of such elements is only capped loosely here.
MAX_BF16_FRAC = 0.05


# Compress paths: the fused single-pass kernel (used whenever the tensor fits
# on chip) and the two-kernel path (larger tensors, or asked for per call).
ENGINES = ["fused", "two_pass", pytest.param("valu", marks=pytest.mark.skip(
    reason="VALU rotation engine removed from libtaco: its compress kernels took a GPU memory "
           "fault on a [3, 1024] tensor (block 64) whose cause was not found"))]


class Mode:
    """The library with compress and decompress_sum_compress taking one pass
    structure per call (single pass where it fits, or always two kernels)."""

    def __init__(self, taco, name):
        if name not in ("fused", "two_pass"):
            pytest.fail(f"no compress path {name!r} in the library")
        self._taco, self.name, self.single_pass = taco, name, name == "fused"

    def __getattr__(self, attr):
        return getattr(self._taco, attr)

    def compress(self, *a, **k):
        k.setdefault("single_pass", self.single_pass)
        return self._taco.compress(*a, **k)

    def decompress_sum_compress(self, *a, **k):
        k.setdefault("single_pass", self.single_pass)
        return self._taco.decompress_sum_compress(*a, **k)

    def two_shot_allreduce(self, *a, **k):
        k.setdefault("single_pass", self.single_pass)
        return self._taco.two_shot_allreduce(*a, **k)


@pytest.fixture(params=ENGINES)
def engine(request, taco):
    return Mode(taco, request.param)


def run_round_trip(taco, bits, block, E=1.0, max_code_frac=1e-4, max_bf16_frac=MAX_BF16_FRAC):
    T, H = bits.shape
    print(f"[case] compress/decompress shape=({T},{H}) block={block} E={E} "
          f"path={getattr(taco, 'name', 'fused')}", flush=True)
    q_o, a_o, s_o = oracle.compress(bits, block, E)
    x = to_gpu_bits(bits)
    q_g, a_g, s_g = gpu_triple_np(*taco.compress(x, block, E))
    parity.check_scales(a_g, s_g, a_o, s_o)
    parity.check_codes(q_g, q_o, bits, a_o, s_o, block, max_frac=max_code_frac)
    # decompress the oracle's triple on the GPU
    trip = (torch.from_numpy(q_o).cuda(), torch.from_numpy(a_o).cuda(),
            torch.tensor([s_o], dtype=torch.float32).cuda())
    xh_g = W.bf16_bits(taco.decompress(*trip, block))
    xh_o = oracle.decompress(q_o, a_o, s_o, block)
    exact = oracle.decompress_f64(q_o, a_o, s_o, block)
    parity.bf16_neighbours_ok(xh_g, xh_o, exact,
                              parity.decompress_error_bound(q_o, a_o, s_o, block), max_bf16_frac)
    # full GPU round trip against the oracle's round trip
    rt = W.bf16_bits(taco.decompress(*[torch.from_numpy(np.atleast_1d(t)).cuda()
                                       for t in (q_g, a_g, s_g)], block))
    assert parity.rel_frobenius(rt, xh_o) <= 1e-3
    return q_g, a_g, s_g


# ------------------------------------------------------------------ small sizes
SMALL = [("tiny", 256), ("tiny", 3), ("gpt2_1p5b", 37), ("gpt3_6p7b_act", 19),
         ("gpt3_6p7b_grad", 21), ("qwen_7b", 23), ("dsum_part", 9)]


@pytest.mark.parametrize("name,tokens", SMALL)
def test_small_round_trip(engine, name, tokens):
    taco = engine
    w = W.WORKLOADS[name]
    bits = W.bf16_bits(W.make(name, seed=5, tokens=tokens))
    run_round_trip(taco, bits, w.block)


@pytest.mark.parametrize("block", [64, 128, 256])
@pytest.mark.parametrize("tokens,hidden", [(1, 256), (5, 768), (131, 512)])
def test_small_shapes_every_block(engine, block, tokens, hidden):
    taco = engine
    rng = np.random.default_rng(tokens * hidden + block)
    vals = rng.standard_normal((tokens, hidden)) * np.exp(rng.uniform(-6, 6, (tokens, 1)))
    run_round_trip(taco, oracle.f64_to_bf16_bits(vals), block)


@pytest.mark.parametrize("E", [1.0, 0.25, 37.5])
def test_target_energy(engine, E):
    taco = engine
    bits = W.bf16_bits(W.make("gpt3_6p7b_act", seed=2, tokens=16))
    run_round_trip(taco, bits, 128, E)


# ------------------------------------------------------------------ edge cases
def test_zero_tensor(engine):
    taco = engine
    bits = np.zeros((4, 256), dtype=np.uint16)
    q, a, s = run_round_trip(taco, bits, 64)
    assert s == 1.0 and np.all(a == 1.0) and np.all(parity.ordinal(q) == 0)


def test_negative_zeros_and_zero_blocks(engine):
    taco = engine
    rng = np.random.default_rng(0)
    vals = rng.standard_normal((8, 512)) * 0.01
    vals[2, :] = -0.0
    vals[5, 128:256] = 0.0
    run_round_trip(taco, oracle.f64_to_bf16_bits(vals), 128)


@pytest.mark.parametrize("block", [64, 128, 256])
def test_one_hot_and_constant_blocks(engine, block):
    taco = engine
    vals = np.zeros((4, 2 * block))
    vals.reshape(-1, block)[0, 3] = 0.75
    vals.reshape(-1, block)[1, block - 1] = -3.0
    vals.reshape(-1, block)[2, :] = 0.5
    vals.reshape(-1, block)[3, :] = -2.0 ** -7
    vals.reshape(-1, block)[4, 0] = 2.0 ** -5
    vals.reshape(-1, block)[5, :] = np.linspace(-1, 1, block)
    vals.reshape(-1, block)[6, ::7] = 1.0
    run_round_trip(taco, oracle.f64_to_bf16_bits(vals), block)


@pytest.mark.parametrize("scale_exp", [-50, -20, 20, 50])
def test_extreme_magnitudes(engine, scale_exp):
    taco = engine
    bits = W.bf16_bits(W.make("tiny", seed=9, tokens=8))
    vals = oracle.bf16_bits_to_f64(bits) * 2.0 ** scale_exp
    q, a, s = run_round_trip(taco, oracle.f64_to_bf16_bits(vals), 64)
    # the GPU arithmetic is exactly invariant under power-of-two input scaling:
    # same codes and s, alpha scaled by the inverse power
    q0, a0, s0 = gpu_triple_np(*taco.compress(to_gpu_bits(bits), 64))
    assert np.array_equal(q, q0) and s == s0
    assert np.array_equal(a, a0 * np.float32(2.0 ** -scale_exp))


def test_every_fp8_code_decodes_exactly(taco):
    """Row r holds code r at position 0 and zeros elsewhere (alpha = s = 1), so
    the decompressed row is decode(r) / sqrt(64) in every position."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q = np.zeros((codes.size, 64), dtype=np.uint8)
    q[:, 0] = codes
    a = np.ones((codes.size, 1), dtype=np.float32)
    out = taco.decompress(torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(),
                          torch.ones(1, dtype=torch.float32).cuda(), 64)
    got = oracle.bf16_bits_to_f64(W.bf16_bits(out))
    want = oracle.e4m3_decode(codes) / 8.0
    assert np.array_equal(got, np.repeat(want[:, None], 64, axis=1))


def _compress_with(taco, x, block, single_pass, ws, polls=0):
    return [t.clone() for t in taco.compress(x, block, workspace=ws, single_pass=single_pass,
                                            barrier_polls=polls)]


def test_fused_matches_two_pass_bitwise(taco):
    """The fused kernel and the two-kernel path evaluate the same arithmetic:
    identical codes, alpha and scale.  The shapes alternate between grids of
    many barrier leaves and of one, on one workspace, so every call must find
    the barrier state the previous call left; the barrier never times out.
    Beyond the fused kernel's capacity the library takes two kernels."""
    nbytes = taco.workspace_bytes(8192, 3584, 128)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    # B <= 128 holding y: x staged through LDS (1, 2 and 4 tiles per wavefront,
    # the two 4095-token shapes with a ragged last tile); the last four hold the
    # bf16 input rather than the rotated blocks, staged through a ring of two
    # LDS tiles (4, 3, 6 and 4 tiles per wavefront; the last with 8 wavefronts
    # per CU)
    cases = [("gpt3_6p7b_act", 4096, 128), ("tiny", 3, 64), ("gpt2_1p5b", 4096, 64),
             ("tiny", 256, 256), ("gpt3_6p7b_grad", 1024, 128), ("dsum_part", 17, 256),
             ("qwen_7b", 4096, 64), ("gpt2_1p5b", 4095, 64), ("qwen_7b", 4095, 128),
             ("gpt3_6p7b_act", 4096, 128), ("qwen_7b", 8192, 128), ("qwen_7b", 5120, 128),
             ("qwen_7b", 6144, 64), ("qwen_7b", 8192, 256),
             # B = 256 holding y through LDS with a ragged last tile (one tile, and 3,584)
             ("tiny", 3, 256), ("qwen_7b", 4095, 256),
             # one tile per wavefront on workgroups of 8, 4 and 16 wavefronts (on
             # 256 CUs: 1,536, 200, 3,125 and 3,072 tiles)
             ("gpt2_1p5b", 983, 64), ("dsum_part", 1536, 256), ("gpt3_6p7b_grad", 100, 128),
             ("gpt2_1p5b", 2000, 64), ("gpt3_6p7b_act", 1536, 128)]
    for name, tokens, block in cases:
        print(f"[case] fused vs two-pass {name} tokens={tokens} block={block}", flush=True)
        x = W.make(name, seed=tokens, tokens=tokens).cuda()
        assert taco.is_single_pass(*x.shape, block)          # the fused kernel really runs
        fused = _compress_with(taco, x, block, True, ws)
        two = _compress_with(taco, x, block, False, ws)
        for a, b in zip(fused, two):
            assert torch.equal(a, b)
        timed_out = int(ws[8:12].cpu().numpy().view(np.uint32)[0])
        assert timed_out == 0
    assert not taco.is_single_pass(8192, 3584, 64)            # 29.4M elements at B = 64
    assert not taco.is_single_pass(16384, 4096, 128)


def _tiles_equal_or_nan(q, ref, block):
    """Per tile of 16 blocks: the codes equal the reference or are all NaN.
    Returns (tiles equal, tiles NaN)."""
    qt = q.reshape(-1, 16 * block)
    rt = ref.reshape(-1, 16 * block)
    eq = (qt == rt).all(dim=1)
    nan = ((qt & 0x7F) == 0x7F).all(dim=1)
    assert bool((eq | nan).all())
    return int(eq.sum()), int(nan.sum())


def test_barrier_timeout_gives_nan_codes_and_keeps_the_workspace(taco):
    """The barrier's bounded wait, forced from the host with a bound of one
    poll: the workgroups that give up store NaN codes (never plausible codes
    under a stale scale), every other tile is exact, alpha is unaffected, the
    sticky flag is set, and the workspace stays valid for the next call."""
    block = 128
    x = W.make("gpt3_6p7b_act", seed=4096, tokens=4096).cuda()
    ref = _compress_with(taco, x, block, False, torch.zeros(taco.workspace_bytes(4096, 4096, block),
                                                             dtype=torch.uint8, device="cuda"))
    ws = torch.zeros(taco.workspace_bytes(4096, 4096, block), dtype=torch.uint8, device="cuda")
    print("[case] fused compress, barrier bound of 1 poll", flush=True)
    q, a, s = _compress_with(taco, x, block, True, ws, polls=1)
    assert taco.workspace_timed_out(ws)
    eq, nan = _tiles_equal_or_nan(q, ref[0], block)
    assert nan >= 1                       # the others may pass or give up too
    assert torch.equal(a, ref[1])
    assert torch.equal(s, ref[2]) or bool(torch.isnan(s).all())
    print("[case] fused compress after the timeout, same workspace", flush=True)
    for r, t in zip(ref, _compress_with(taco, x, block, True, ws)):
        assert torch.equal(r, t)
    assert taco.workspace_timed_out(ws)                 # sticky until zero-filled
    ws.zero_()
    assert not taco.workspace_timed_out(ws)
    for r, t in zip(ref, _compress_with(taco, x, block, True, ws)):
        assert torch.equal(r, t)
    assert not taco.workspace_timed_out(ws)

    print("[case] fused decompress-sum-compress, barrier bound of 1 poll", flush=True)
    parts = [taco.compress(W.make("gpt3_6p7b_act", seed=40 + i, tokens=4096).cuda(), block)
             for i in range(2)]
    parts = [tuple(t.clone() for t in p) for p in parts]
    ws2 = torch.zeros(taco.load().taco_decompress_sum_compress_workspace_bytes(4096, 4096, block),
                      dtype=torch.uint8, device="cuda")
    ref2 = [t.clone() for t in taco.decompress_sum_compress(parts, block, workspace=ws2)]
    assert not taco.workspace_timed_out(ws2)
    q2, a2, s2 = [t.clone() for t in taco.decompress_sum_compress(parts, block, workspace=ws2,
                                                                 barrier_polls=1)]
    assert taco.workspace_timed_out(ws2)
    eq, nan = _tiles_equal_or_nan(q2, ref2[0], block)
    assert nan >= 1                       # the others may pass or give up too
    assert torch.equal(a2, ref2[1])
    for r, t in zip(ref2, taco.decompress_sum_compress(parts, block, workspace=ws2)):
        assert torch.equal(r, t)


def test_barrier_timeout_fallback_gives_the_exact_result(taco):
    """The host-side fallback the header documents (check_barrier=True): after
    a single-pass call whose workgroups gave up at the barrier (a bound of one
    poll forces it), the flag is cleared and the call is repeated with the two
    kernels, so the caller gets the exact result and a clean workspace."""
    block = 128
    x = W.make("gpt3_6p7b_act", seed=4097, tokens=4096).cuda()
    ref = _compress_with(taco, x, block, False, torch.zeros(taco.workspace_bytes(4096, 4096, block),
                                                             dtype=torch.uint8, device="cuda"))
    ws = torch.zeros(taco.workspace_bytes(4096, 4096, block), dtype=torch.uint8, device="cuda")
    print("[case] fused compress with the checked fallback, bound of 1 poll", flush=True)
    got = [t.clone() for t in taco.compress(x, block, workspace=ws, barrier_polls=1, check_barrier=True)]
    for r, t in zip(ref, got):
        assert torch.equal(r, t)
    assert not taco.workspace_timed_out(ws)
    parts = [tuple(t.clone() for t in taco.compress(W.make("gpt3_6p7b_act", seed=50 + i, tokens=4096).cuda(),
                                                     block)) for i in range(3)]
    ws2 = torch.zeros(taco.load().taco_decompress_sum_compress_workspace_bytes(4096, 4096, block),
                      dtype=torch.uint8, device="cuda")
    ref2 = [t.clone() for t in taco.decompress_sum_compress(parts, block, workspace=ws2, single_pass=False)]
    print("[case] fused decompress-sum-compress with the checked fallback, bound of 1 poll", flush=True)
    got2 = [t.clone() for t in taco.decompress_sum_compress(parts, block, workspace=ws2, barrier_polls=1,
                                                             check_barrier=True)]
    for r, t in zip(ref2, got2):
        assert torch.equal(r, t)
    assert not taco.workspace_timed_out(ws2)


# The barrier's workspace layout, as the kernels define it: a 256-byte root
# line (the timed-out flag at byte 8), 64 leaf lines of 256 bytes whose first
# 8 bytes are a running count, 1024 partial maxima of 4 bytes, then 1024 slots
# of 16 bytes whose first 8 hold (epoch << 32) | max bits.
LEAF0, LINE, LEAVES = 256, 256, 64
SLOT0, SLOT_STRIDE, SLOTS = 256 * 65 + 4 * 1024, 16, 1024


def _preset_barrier(ws, calls):
    """Writes the barrier state that `calls` calls leave: every leaf count at
    16 * calls and every slot at epoch `calls` (its low 32 bits)."""
    w = ws[:SLOT0 + SLOT_STRIDE * SLOTS].cpu().numpy().copy()
    for l in range(LEAVES):
        w[LEAF0 + LINE * l:LEAF0 + LINE * l + 8].view(np.uint64)[0] = np.uint64(16 * calls)
    slots = w[SLOT0:].view(np.uint64).reshape(SLOTS, 2)
    slots[:, 0] = np.uint64((calls & 0xFFFFFFFF) << 32)
    ws[:w.size].copy_(torch.from_numpy(w))


@pytest.mark.parametrize("calls", [(1 << 27) - 1, (1 << 28) - 1])
def test_barrier_counts_cross_bit_31_and_bit_32(taco, calls):
    """The leaf counts are 64-bit and never reset.  From the state after
    2^27 - 1 (2^28 - 1) calls, the next call takes the low word of the counts
    across 2^31 (2^32) and the later ones run beyond it: every workgroup
    still derives the same epoch from its count, so no poll gives up and
    the results equal a fresh workspace's, for a kernel holding y, one
    holding x and the fused decompress-sum-compress.  (The count was once
    widened from a signed 32-bit half, which gave the workgroups that read a
    count with bit 31 set another epoch.)"""
    block = 128
    for name, tokens, hidden in [("gpt3_6p7b_act", 4096, 4096), ("qwen_7b", 8192, 3584)]:
        x = W.make(name, seed=31, tokens=tokens).cuda()
        assert taco.is_single_pass(tokens, hidden, block)
        ref = _compress_with(taco, x, block, True, torch.zeros(taco.workspace_bytes(tokens, hidden, block),
                                                                dtype=torch.uint8, device="cuda"))
        ws = torch.zeros(taco.workspace_bytes(tokens, hidden, block), dtype=torch.uint8, device="cuda")
        _preset_barrier(ws, calls)
        for k in range(3):
            print(f"[case] {name} compress, call {calls + k} of a preset workspace", flush=True)
            for r, t in zip(ref, _compress_with(taco, x, block, True, ws)):
                assert torch.equal(r, t)
            assert not taco.workspace_timed_out(ws)
    parts = [tuple(t.clone() for t in taco.compress(W.make("gpt3_6p7b_act", seed=60 + i, tokens=4096).cuda(),
                                                     block)) for i in range(2)]
    nbytes = taco.load().taco_decompress_sum_compress_workspace_bytes(4096, 4096, block)
    ref2 = [t.clone() for t in taco.decompress_sum_compress(
        parts, block, workspace=torch.zeros(nbytes, dtype=torch.uint8, device="cuda"))]
    ws2 = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    _preset_barrier(ws2, calls)
    for k in range(3):
        print(f"[case] decompress-sum-compress, call {calls + k} of a preset workspace", flush=True)
        got = [t.clone() for t in taco.decompress_sum_compress(parts, block, workspace=ws2)]
        for r, t in zip(ref2, got):
            assert torch.equal(r, t)
        assert not taco.workspace_timed_out(ws2)


def test_barrier_over_many_calls_on_one_workspace(taco):
    """2000 single-pass calls on one workspace, cycling through grids of 16,
    200, 256 and 224 workgroups (y held at B = 64 and 128, x held at
    B = 128): every result bitwise equal to the same call on a fresh
    workspace, and no poll ever gives up."""
    cases = [("tiny", 256, 64), ("gpt2_1p5b", 4096, 64), ("gpt3_6p7b_act", 4096, 128), ("qwen_7b", 8192, 128)]
    xs, refs = [], []
    for name, tokens, block in cases:
        x = W.make(name, seed=90, tokens=tokens).cuda()
        assert taco.is_single_pass(*x.shape, block)
        fresh = torch.zeros(taco.workspace_bytes(*x.shape, block), dtype=torch.uint8, device="cuda")
        xs.append((x, block))
        refs.append(_compress_with(taco, x, block, True, fresh))
    ws = torch.zeros(taco.workspace_bytes(8192, 3584, 128), dtype=torch.uint8, device="cuda")
    print("[case] 2000 fused compress calls on one workspace", flush=True)
    outs = [[torch.empty_like(t) for t in r] for r in refs]
    for it in range(500):
        for k, (x, block) in enumerate(xs):
            q, a, s = outs[k]
            taco.compress(x, block, q=q, alpha=a, scale=s, workspace=ws)
            if it % 50 == 49 or it == 0:
                for r, t in zip(refs[k], outs[k]):
                    assert torch.equal(r, t), (it, cases[k])
    for k in range(len(xs)):
        for r, t in zip(refs[k], outs[k]):
            assert torch.equal(r, t)
    assert not taco.workspace_timed_out(ws)


def test_determinism(engine):
    taco = engine
    x = W.make("gpt2_1p5b", seed=3, tokens=512).cuda()
    r1 = [t.clone() for t in taco.compress(x, 64)]
    for _ in range(20):
        r2 = taco.compress(x, 64)
        for a, b in zip(r1, r2):
            assert torch.equal(a, b)


# ------------------------------------------------------------------ decompress-sum
def run_decompress_sum(taco, part_bits, block):
    T, H = part_bits[0].shape
    print(f"[case] decompress_sum parts={len(part_bits)} shape=({T},{H}) block={block}", flush=True)
    trip_o = [oracle.compress(b, block) for b in part_bits]
    ref = oracle.decompress_sum(trip_o, block)
    exact = sum(oracle.decompress_f64(*t, block) for t in trip_o)
    gpu_parts = [(torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(),
                  torch.tensor([s], dtype=torch.float32).cuda()) for q, a, s in trip_o]
    got = W.bf16_bits(taco.decompress_sum(gpu_parts, block))
    parity.bf16_neighbours_ok(got, ref, exact, parity.decompress_sum_error_bound(trip_o, block),
                              MAX_BF16_FRAC)
    assert parity.rel_frobenius(got, ref) <= 1e-3
    # the GPU's own compressions summed on the GPU, against the oracle's sum
    mine = [taco.compress(to_gpu_bits(b), block) for b in part_bits]
    got2 = W.bf16_bits(taco.decompress_sum(mine, block))
    assert parity.rel_frobenius(got2, ref) <= 1e-3


@pytest.mark.parametrize("nparts", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decompress_sum_small(taco, nparts):
    parts = [W.bf16_bits(W.make("dsum_part", seed=p, tokens=7)) for p in range(nparts)]
    run_decompress_sum(taco, parts, 256)


@pytest.mark.parametrize("block", [64, 128])
def test_decompress_sum_other_blocks(taco, block):
    parts = [W.bf16_bits(W.make("gpt3_6p7b_act", seed=p, tokens=11)) for p in range(4)]
    run_decompress_sum(taco, parts, block)


def test_decompress_sum_one_part_matches_decompress(taco):
    """One part: the same reconstruction as decompress, up to the fp32 rounding
    order (the sum applies 1/(alpha s) before the rotation, decompress after)."""
    bits = W.bf16_bits(W.make("gpt3_6p7b_act", seed=1, tokens=64))
    q, a, s = oracle.compress(bits, 128)
    t = (torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(),
         torch.tensor([s], dtype=torch.float32).cuda())
    one = W.bf16_bits(taco.decompress_sum([t], 128))
    ref = oracle.decompress(q, a, s, 128)
    exact = oracle.decompress_f64(q, a, s, 128)
    parity.bf16_neighbours_ok(one, ref, exact, parity.decompress_sum_error_bound([(q, a, s)], 128),
                              MAX_BF16_FRAC)
    assert parity.rel_frobenius(one, W.bf16_bits(taco.decompress(*t, 128))) <= 1e-3


# ------------------------------------------------------------------ full sizes
FULL = ["tiny", "gpt2_1p5b", "gpt3_6p7b_act", "gpt3_6p7b_grad", "qwen_7b"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_round_trip(engine, name):
    taco = engine
    w = W.WORKLOADS[name]
    seed = 1 if name == "gpt3_6p7b_grad" else 0
    bits = W.bf16_bits(W.make(name, seed=seed))
    run_round_trip(taco, bits, w.block)


@pytest.mark.parametrize("tokens,block", [(4096, 64), (4095, 128)])
def test_lds_staged_fused_against_oracle(taco, tokens, block):
    """The fused compress that copies x into LDS at its larger configurations,
    element by element against the oracle: [4096, 3584] at B = 64 runs four
    tiles per wavefront, [4095, 3584] at B = 128 two with a ragged last tile."""
    assert taco.is_single_pass(tokens, 3584, block)
    bits = W.bf16_bits(W.make("qwen_7b", seed=7, tokens=tokens))
    run_round_trip(taco, bits, block)


def test_full_size_decompress_sum_32_layers(taco):
    """4 parts of [4096, 4096] at block 256; the same call repeated over 32
    layer slots gives bitwise-identical outputs."""
    parts = [W.bf16_bits(W.make("dsum_part", seed=p)) for p in range(4)]
    run_decompress_sum(taco, parts, 256)
    gp = [taco.compress(to_gpu_bits(b), 256) for b in parts]
    outs = [taco.decompress_sum(gp, 256) for _ in range(32)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


# ------------------------------------------------------------------ decompress-sum-compress
def run_decompress_sum_compress(taco, part_bits, block, E=1.0):
    """compress(decompress_sum(parts)) in one call.

    (a) Bitwise equal to the two GPU calls in sequence, each of which meets its
    own element-wise parity bars against the oracle in the tests above.
    (b) Against the oracle's composition directly.  The GPU's fp32 sum can round
    to a different bf16 value than the oracle's fp64 sum, by one ulp near a
    tie and by several where the parts cancel (the sum's error scales with the
    sum of the parts' magnitudes, not with the result), and such an element
    changes the rotated values of its whole block.  So: every differing element
    of the sum must be a bf16 tie within the fp32 error bound (as in the
    decompress-sum tests); the full bars apply to every block whose bf16 sum
    equals the oracle's bitwise (the same input to the compression): alpha
    within 1e-6, and codes at most 1e-4 off, each by at most one step at a
    rounding tie; s is held to 1e-6 whenever the block holding the oracle's
    maximum is such a block and no block with a differing sum can reach that
    maximum (an upper bound from its differing elements), otherwise to 2^-7.
    Blocks with a different bf16 sum: alpha within 2^-6; all blocks:
    reconstructions within 1e-3 relative Frobenius."""
    T, H = part_bits[0].shape
    print(f"[case] decompress_sum_compress parts={len(part_bits)} shape=({T},{H}) block={block} "
          f"path={getattr(taco, 'name', 'fused')}", flush=True)
    trip_o = [oracle.compress(b, block) for b in part_bits]
    gparts = [(torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(),
               torch.tensor([s], dtype=torch.float32).cuda()) for q, a, s in trip_o]
    got = [t.clone() for t in taco.decompress_sum_compress(gparts, block, E)]
    comp = taco.compress(taco.decompress_sum(gparts, block), block, E)
    for a, b in zip(got, comp):
        assert torch.equal(a, b)
    q_g, a_g, s_g = gpu_triple_np(*got)
    q_o, a_o, s_o = oracle.decompress_sum_compress(trip_o, block, E)
    sum_o = oracle.decompress_sum(trip_o, block)                  # the oracle's bf16 sum
    sum_g = W.bf16_bits(taco.decompress_sum(gparts, block))       # the fused kernel's input
    # every element of the GPU's sum that differs from the oracle's is the
    # neighbouring bf16 value at a rounding tie within the fp32 error bound
    exact = sum(oracle.decompress_f64(*t, block) for t in trip_o)
    parity.bf16_neighbours_ok(sum_g, sum_o, exact, parity.decompress_sum_error_bound(trip_o, block),
                              MAX_BF16_FRAC)
    diff = (sum_o != sum_g).reshape(-1, block)
    same = ~np.any(diff, axis=1)
    rel_a = (np.abs(a_g.astype(np.float64) - a_o) / a_o).reshape(-1)
    assert np.max(rel_a[same], initial=0.0) <= 1e-6
    assert np.max(rel_a, initial=0.0) <= 2.0 ** -6
    assert np.mean(same) >= 0.5, f"only {np.mean(same):.3f} of the blocks have the oracle's bf16 sum"
    # s: the oracle's max |y| per block, and for the blocks whose sum differs an
    # upper bound on the GPU's: each differing element moves by one bf16 step,
    # at most 2^-7 |x_i|, so max|H x| grows by at most |d|_1 and |x|_2 shrinks
    # by at most |d|_2 (alpha = sqrt(E B) / |x|_2).
    xb = oracle.bf16_bits_to_f64(sum_o).reshape(-1, block)
    bmax = np.max(np.abs(oracle.hadamard_rotate(xb, a_o.reshape(-1))), axis=1)
    d = 2.0 ** -7 * np.abs(xb) * diff
    hx = np.max(np.abs(xb @ oracle.hadamard(block).T), axis=1)
    nx = np.linalg.norm(xb, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        bound = np.sqrt(E) * (hx + d.sum(axis=1)) / (nx - np.linalg.norm(d, axis=1))
    A = np.max(bmax)
    rel_s = abs(float(s_g) - float(s_o)) / float(s_o)
    full = A > 0 and bool(same[np.argmax(bmax)]) and bool(np.all(bound[~same] < A * (1 - 2e-6)))
    print(f"[case]   blocks with the oracle's bf16 sum: {np.mean(same):.4f}; "
          f"the maximum's block is one of them and no other can reach it: {full}; rel s {rel_s:.2e}",
          flush=True)
    if full or A == 0:
        assert rel_s <= 1e-6
        parity.check_codes(q_g.reshape(-1, block)[same], q_o.reshape(-1, block)[same],
                           sum_o.reshape(-1, block)[same], a_o.reshape(-1)[same], s_o, block)
    else:
        assert rel_s <= 2.0 ** -7
    xh_g = W.bf16_bits(taco.decompress(*got, block))
    xh_o = oracle.decompress(q_o, a_o, s_o, block)
    assert parity.rel_frobenius(xh_g, xh_o) <= 1e-3
    return got


@pytest.mark.parametrize("nparts", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decompress_sum_compress_small(engine, nparts):
    taco = engine
    parts = [W.bf16_bits(W.make("dsum_part", seed=p, tokens=7)) for p in range(nparts)]
    run_decompress_sum_compress(taco, parts, 256)


@pytest.mark.parametrize("block", [64, 128])
def test_decompress_sum_compress_other_blocks(engine, block):
    taco = engine
    parts = [W.bf16_bits(W.make("gpt3_6p7b_act", seed=p, tokens=11)) for p in range(4)]
    run_decompress_sum_compress(taco, parts, block, 0.5)


def test_decompress_sum_compress_zero_sum(engine):
    taco = engine
    bits = W.bf16_bits(W.make("gpt3_6p7b_act", seed=3, tokens=5))
    q, a, s = oracle.compress(bits, 128)
    neg = (q ^ np.uint8(0x80), a, s)
    gparts = [(torch.from_numpy(t[0]).cuda(), torch.from_numpy(t[1]).cuda(),
               torch.tensor([t[2]], dtype=torch.float32).cuda()) for t in [(q, a, s), neg]]
    qz, az, sz = gpu_triple_np(*taco.decompress_sum_compress(gparts, 128))
    assert sz == 1.0 and np.all(az == 1.0) and np.all(parity.ordinal(qz) == 0)


def test_decompress_sum_compress_two_tiles_per_wavefront_b64(taco):
    """4 parts of [4096, 1600] at block 64: 6400 tiles, more than one tile per
    wavefront fits on one workgroup per CU, so the fused kernel runs two
    tiles per wavefront (200 workgroups); checked bitwise against the
    two-kernel path and against the oracle."""
    parts = [W.bf16_bits(W.make("gpt2_1p5b", seed=70 + p)) for p in range(4)]
    ws = torch.zeros(taco.load().taco_decompress_sum_compress_workspace_bytes(4096, 1600, 64),
                     dtype=torch.uint8, device="cuda")
    trip = [oracle.compress(b, 64) for b in parts]
    gparts = [(torch.from_numpy(q).cuda(), torch.from_numpy(a).cuda(),
               torch.tensor([s], dtype=torch.float32).cuda()) for q, a, s in trip]
    got = [t.clone() for t in taco.decompress_sum_compress(gparts, 64, workspace=ws)]
    assert not taco.workspace_timed_out(ws)
    two = taco.decompress_sum_compress(gparts, 64, single_pass=False)
    for a, b in zip(got, two):
        assert torch.equal(a, b)
    run_decompress_sum_compress(taco, parts, 64)


def test_full_size_decompress_sum_compress(engine):
    taco = engine
    """The decompress-sum workload (4 parts of [4096, 4096], block 256)."""
    parts = [W.bf16_bits(W.make("dsum_part", seed=p)) for p in range(4)]
    run_decompress_sum_compress(taco, parts, 256)


# ------------------------------------------------------------ Dual-Scale variants
def run_blockscale(taco, bits, block, E):
    T, H = bits.shape
    print(f"[case] compress_blockscale shape=({T},{H}) block={block} E={E}", flush=True)
    q_o, a_o, s_o = oracle.compress_blockscale(bits, block, E)
    q_g, a_g, s_g = [t.cpu().numpy() for t in taco.compress_blockscale(to_gpu_bits(bits), block, E)]
    parity.check_scales(a_g, 1.0, a_o, 1.0)
    rel_s = np.abs(s_g.astype(np.float64) - s_o) / s_o
    assert np.max(rel_s) <= 1e-6
    parity.check_codes(q_g, q_o, bits, a_o, s_o, block)
    trip = [torch.from_numpy(t).cuda() for t in (q_o, a_o, s_o)]
    xh_g = W.bf16_bits(taco.decompress_blockscale(*trip, block))
    xh_o = oracle.decompress_blockscale(q_o, a_o, s_o, block)
    exact = oracle.decompress_blockscale_f64(q_o, a_o, s_o, block)
    parity.bf16_neighbours_ok(xh_g, xh_o, exact, parity.decompress_error_bound(q_o, a_o, s_o, block),
                              MAX_BF16_FRAC)
    return q_g, a_g, s_g


@pytest.mark.parametrize("E", [1.0, 2.0 ** 12, 2.0 ** 16])
@pytest.mark.parametrize("name,tokens", [("tiny", 3), ("gpt2_1p5b", 37), ("gpt3_6p7b_act", 19),
                                         ("dsum_part", 9)])
def test_blockscale_small(taco, name, tokens, E):
    w = W.WORKLOADS[name]
    run_blockscale(taco, W.bf16_bits(W.make(name, seed=4, tokens=tokens)), w.block, E)


def test_blockscale_overflowing_blocks_reach_448(taco):
    bits = W.bf16_bits(W.make("gpt3_6p7b_act", seed=6, tokens=8))
    q, a, s = run_blockscale(taco, bits, 128, 2.0 ** 16)
    over = s.reshape(-1) < 1.0
    assert over.any()
    assert np.all(np.max(parity.ordinal(q).reshape(-1, 128)[over] ** 2, axis=1) == 126 ** 2)


@pytest.mark.parametrize("name", ["gpt3_6p7b_act", "qwen_7b"])
def test_full_size_blockscale(taco, name):
    w = W.WORKLOADS[name]
    run_blockscale(taco, W.bf16_bits(W.make(name, seed=0)), w.block, 1.0)


def run_delayed(taco, bits, block, E, amax_prev_value):
    """One delayed-scale call with amax_prev holding amax_prev_value in slot 0;
    the oracle gets the same value."""
    T, H = bits.shape
    print(f"[case] compress_delayed shape=({T},{H}) block={block} amax_prev={amax_prev_value}", flush=True)
    prev = torch.zeros(taco.TACO_AMAX_FLOATS, dtype=torch.float32, device="cuda")
    prev[0] = amax_prev_value
    q_o, a_o, s_o, A_o = oracle.compress_delayed(bits, block, E, amax_prev_value)
    q_g, a_g, s_g, amax = taco.compress_delayed(to_gpu_bits(bits), block, prev, E)
    q_g, a_g, s_g = gpu_triple_np(q_g, a_g, s_g)
    assert s_g == s_o                           # the same fp32 division on both sides
    parity.check_scales(a_g, s_g, a_o, s_o)
    parity.check_codes(q_g, q_o, bits, a_o, s_o, block)
    A_g = float(amax.max().cpu())
    assert abs(A_g - A_o) <= 1e-6 * A_o
    xh_g = W.bf16_bits(taco.decompress(*[torch.from_numpy(np.atleast_1d(t)).cuda()
                                         for t in (q_g, a_g, s_g)], block))
    xh_o = oracle.decompress(q_o, a_o, s_o, block)
    assert parity.rel_frobenius(xh_g, xh_o) <= 1e-3
    return A_o


@pytest.mark.parametrize("name,tokens", [("tiny", 3), ("gpt2_1p5b", 37), ("gpt3_6p7b_grad", 21),
                                         ("dsum_part", 9)])
def test_delayed_small_sequence(taco, name, tokens):
    """No history (s = 1), then the first call's maximum (the oracle's, as fp32),
    then a quarter of it (saturation)."""
    w = W.WORKLOADS[name]
    bits = W.bf16_bits(W.make(name, seed=8, tokens=tokens))
    A = run_delayed(taco, bits, w.block, 1.0, 0.0)
    run_delayed(taco, bits, w.block, 1.0, float(np.float32(A)))
    run_delayed(taco, bits, w.block, 1.0, float(np.float32(A / 4)))


@pytest.mark.parametrize("block", [64, 128, 256])
def test_dual_scale_variants_edge_cases(taco, block):
    """Zero tensors, one-hot and constant blocks, and power-of-two magnitudes
    for the per-block guard and the delayed scale, each against the oracle;
    scaling x by 2^+-50 must scale alpha by 2^-+50 and leave codes and s_k
    bitwise unchanged."""
    H = 4 * block
    zero = np.zeros((3, H), dtype=np.uint16)
    run_blockscale(taco, zero, block, 1.0)
    run_delayed(taco, zero, block, 1.0, 0.0)
    x = np.zeros((2, H))
    x[0, 5] = 3.0
    x[0, block:2 * block] = -0.75
    x[1, 2 * block + 7] = -2.0 ** -20
    x[1, 3 * block:] = 1e-3
    bits = oracle.f64_to_bf16_bits(x)
    for E in (1.0, 2.0 ** 16):
        run_blockscale(taco, bits, block, E)
    run_delayed(taco, bits, block, 1.0, 1.0)
    base = np.ascontiguousarray(W.bf16_bits(W.make("tiny", seed=2, tokens=4))[:, :H])
    q0, a0, s0 = run_blockscale(taco, base, block, 1.0)
    for e in (-50, 50):
        xs = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f64(base) * 2.0 ** e)
        q1, a1, s1 = run_blockscale(taco, xs, block, 1.0)
        assert np.array_equal(q1, q0) and np.array_equal(s1, s0)
        assert np.array_equal(a1, (a0.astype(np.float64) * 2.0 ** -e).astype(np.float32))


def test_delayed_amax_out_accumulates(taco):
    """amax_out keeps the max of its content and this call's block maxima."""
    bits = W.bf16_bits(W.make("tiny", seed=1, tokens=64))
    x = to_gpu_bits(bits)
    out = torch.full((taco.TACO_AMAX_FLOATS,), 1e30, dtype=torch.float32, device="cuda")
    taco.compress_delayed(x, 64, None, 1.0, amax_out=out)
    assert torch.all(out == 1e30)
    out.zero_()
    taco.compress_delayed(x, 64, None, 1.0, amax_out=out)
    _, _, _, A = oracle.compress_delayed(bits, 64, 1.0, 0.0)
    assert abs(float(out.max().cpu()) - A) <= 1e-6 * A


def test_full_size_delayed(taco):
    w = W.WORKLOADS["gpt3_6p7b_act"]
    bits = W.bf16_bits(W.make("gpt3_6p7b_act", seed=0))
    _, _, _, A = oracle.compress_delayed(bits, w.block, 1.0, 0.0)
    run_delayed(taco, bits, w.block, 1.0, float(np.float32(A)))


# ------------------------------------------------------------ two-shot all-reduce emulation
def run_two_shot(taco, xs_bits, block):
    P = len(xs_bits)
    T, H = xs_bits[0].shape
    print(f"[case] two_shot_allreduce P={P} shape=({T},{H}) block={block}", flush=True)
    got = W.bf16_bits(taco.two_shot_allreduce([to_gpu_bits(b) for b in xs_bits], block))
    want, _ = oracle.two_shot_allreduce(xs_bits, block)
    # two codec stages in sequence, each within 1e-3 of the oracle's
    # reconstruction, so the chain within 2e-3
    assert parity.rel_frobenius(got, want) <= 2e-3
    exact = sum(oracle.bf16_bits_to_f64(b) for b in xs_bits)
    err_g = np.linalg.norm(oracle.bf16_bits_to_f64(got) - exact) / np.linalg.norm(exact)
    err_o = np.linalg.norm(oracle.bf16_bits_to_f64(want) - exact) / np.linalg.norm(exact)
    print(f"[case]   error vs the exact sum: GPU {err_g:.5f} oracle {err_o:.5f}", flush=True)
    assert abs(err_g - err_o) <= 0.05 * err_o + 1e-6


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_two_shot_allreduce_small(engine, P):
    taco = engine
    xs = [W.bf16_bits(W.make("gpt3_6p7b_act", seed=20 + r, tokens=8 * P)) for r in range(P)]
    run_two_shot(taco, xs, 128)


def test_full_size_two_shot_allreduce(taco):
    """4 ranks' [4096, 4096] activations at block 128: 1024-row shards."""
    xs = [W.bf16_bits(W.make("gpt3_6p7b_act", seed=30 + r)) for r in range(4)]
    run_two_shot(taco, xs, 128)


# ------------------------------------------------------------ HIP graphs
def test_graph_replays_match_eager(taco):
    """Every entry point captured in one HIP graph (torch.cuda.CUDAGraph) and
    replayed several times, with eager calls on the same workspaces between the
    replays: every replay reproduces the eager results bitwise (the barrier
    state carries over between calls by design)."""
    T, H, B = 512, 4096, 128
    dev = torch.device("cuda")
    x1 = W.make("gpt3_6p7b_act", seed=11, tokens=T).to(dev)
    x2 = W.make("gpt3_6p7b_grad", seed=12, tokens=T).to(dev)
    ws = torch.zeros(taco.workspace_bytes(T, H, B), dtype=torch.uint8, device=dev)
    ws2 = torch.zeros(taco.load().taco_decompress_sum_compress_workspace_bytes(T, H, B),
                      dtype=torch.uint8, device=dev)
    nb = T * H // B
    out = {
        "q1": torch.empty((T, H), dtype=torch.uint8, device=dev),
        "a1": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "s1": torch.empty(1, dtype=torch.float32, device=dev),
        "q2": torch.empty((T, H), dtype=torch.uint8, device=dev),
        "a2": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "s2": torch.empty(1, dtype=torch.float32, device=dev),
        "xh": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        "sum": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        "rq": torch.empty((T, H), dtype=torch.uint8, device=dev),
        "ra": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "rs": torch.empty(1, dtype=torch.float32, device=dev),
        "bq": torch.empty((T, H), dtype=torch.uint8, device=dev),
        "ba": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "bs": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "dq": torch.empty((T, H), dtype=torch.uint8, device=dev),
        "da": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "ds": torch.empty(1, dtype=torch.float32, device=dev),
        "amax": torch.zeros(taco.TACO_AMAX_FLOATS, dtype=torch.float32, device=dev),
        "prev": torch.zeros(taco.TACO_AMAX_FLOATS, dtype=torch.float32, device=dev),
        "bx": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        "iq": torch.empty((T, H), dtype=torch.int8, device=dev),
        "is": torch.empty(1, dtype=torch.float32, device=dev),
        "ix": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
        "ibq": torch.empty((T, H), dtype=torch.int8, device=dev),
        "ibs": torch.empty((T, H // B), dtype=torch.float32, device=dev),
        "ibx": torch.empty((T, H), dtype=torch.bfloat16, device=dev),
    }
    out["prev"][0] = 3.0

    def ops():
        taco.compress(x1, B, q=out["q1"], alpha=out["a1"], scale=out["s1"], workspace=ws)
        taco.compress(x2, B, q=out["q2"], alpha=out["a2"], scale=out["s2"], workspace=ws)
        taco.decompress(out["q1"], out["a1"], out["s1"], B, out=out["xh"])
        parts = [(out["q1"], out["a1"], out["s1"]), (out["q2"], out["a2"], out["s2"])]
        taco.decompress_sum(parts, B, out=out["sum"])
        taco.decompress_sum_compress(parts, B, q=out["rq"], alpha=out["ra"], scale=out["rs"], workspace=ws2)
        taco.compress_blockscale(x2, B, 2.0 ** 12, q=out["bq"], alpha=out["ba"], scale=out["bs"])
        taco.decompress_blockscale(out["bq"], out["ba"], out["bs"], B, out=out["bx"])
        taco.compress_int8(x1, 0, q=out["iq"], scale=out["is"], workspace=ws)
        taco.decompress_int8(out["iq"], out["is"], 0, out=out["ix"])
        taco.compress_int8(x2, B, q=out["ibq"], scale=out["ibs"])
        taco.decompress_int8(out["ibq"], out["ibs"], B, out=out["ibx"])
        out["amax"].zero_()
        taco.compress_delayed(x1, B, out["prev"], q=out["dq"], alpha=out["da"], scale=out["ds"],
                              amax_out=out["amax"])

    ops()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops()
    for rep in range(4):
        for v in out.values():
            if v.dtype in (torch.uint8, torch.int8):
                v.fill_(0x55)
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(out[k], eager[k]), (rep, k)
        # eager work between the replays, on the same workspaces
        taco.compress(x2, B, workspace=ws)
        taco.decompress_sum_compress([(eager["q2"], eager["a2"], eager["s2"])], B, workspace=ws2)
        torch.cuda.synchronize()
    assert int(ws[8:12].cpu().numpy().view(np.uint32)[0]) == 0
    assert int(ws2[8:12].cpu().numpy().view(np.uint32)[0]) == 0


def test_default_workspaces_are_per_stream(taco):
    """Calls on two streams with the binding's default workspaces run
    concurrently without sharing state: both results equal the single-stream
    ones bitwise.  Two-kernel path: each call's statistics kernel writes the
    partial maxima its quantisation kernel reads, so one workspace shared by
    the two streams would mix them.  (Single-pass calls may not run
    concurrently at all: each needs every compute unit for its barrier.)"""
    xa = W.make("gpt3_6p7b_act", seed=21).cuda()
    xb = W.make("gpt3_6p7b_grad", seed=22).cuda()
    ref_a = [t.clone() for t in taco.compress(xa, 128, single_pass=False)]
    ref_b = [t.clone() for t in taco.compress(xb, 128, single_pass=False)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        # the calls allocate their outputs on the stream they run on
        oa = taco.compress(xa, 128, stream=s1, single_pass=False)
        ob = taco.compress(xb, 128, stream=s2, single_pass=False)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        for r, t in zip(ref_a, oa):
            assert torch.equal(r, t)
        for r, t in zip(ref_b, ob):
            assert torch.equal(r, t)
