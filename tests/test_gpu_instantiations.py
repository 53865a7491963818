"""GPU coverage of every compiled variant of the part-count-templated kernels.

The decompress-sum and the fused decompress-sum-compress are compiled once
per part count (1-8), and the fused kernel also per block size and tiles per
wavefront, which the library picks from the tensor's size.  Each variant is
its own code (its own prefetch depth and unrolled steps), so each is run
here:

* decompress-sum at B = 64 and 128 for every part count, against the oracle
  (B = 256 is covered the same way in test_gpu_parity.py);
* the fused decompress-sum-compress for every (block, tiles per wavefront,
  wavefronts per workgroup, part count) it is compiled for, on random valid
  codes, bitwise against the two-kernel composition (decompress-sum, then
  compress), with a check that the fused kernel ran (it leaves the
  workspace's bf16 intermediate untouched, which the two-kernel path
  writes).
"""
import numpy as np
import pytest
import torch

from fp8_compression_tensor_taco_amd import workloads as W
from test_gpu_parity import run_decompress_sum

pytestmark = pytest.mark.gpu

COMPRESS_WORKSPACE = 37120   # barrier state and partial maxima, before the intermediate
# The library's fused configurations (tiles per wavefront, wavefronts per
# workgroup) in the order it tries them; it takes the first whose grid of
# one workgroup per CU holds every tile.
ORDER = {64: [(1, 4), (1, 8), (1, 16), (2, 16), (4, 16)],
         128: [(1, 4), (1, 8), (1, 16), (2, 16)],
         256: [(2, 8)]}


@pytest.fixture(scope="module")
def taco():
    assert torch.cuda.is_available(), "GPU tests need a GPU (no CPU fallback exists)"
    import fp8_compression_tensor_taco_amd as taco
    taco.load()
    return taco


@pytest.mark.parametrize("block", [64, 128])
@pytest.mark.parametrize("nparts", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decompress_sum_every_part_count(taco, block, nparts):
    parts = [W.bf16_bits(W.make("gpt3_6p7b_act", seed=40 + p, tokens=5)) for p in range(nparts)]
    run_decompress_sum(taco, parts, block)


def shape_for(block, tpw, waves, cus):
    """A [tokens, hidden] whose tile count selects exactly the configuration
    (tpw tiles per wavefront, `waves` wavefronts per workgroup): more tiles
    than the previous configuration in ORDER holds, at most what this one
    does."""
    per_tile = 16 * block
    k = ORDER[block].index((tpw, waves))
    lo = cus * ORDER[block][k - 1][0] * ORDER[block][k - 1][1] if k > 0 else 0
    hi = cus * tpw * waves
    tiles = (lo + hi) // 2 + 3          # strictly inside, and not a multiple of the grid
    hidden = 4096 if block < 256 else 8192
    tokens = -(-tiles * per_tile // hidden)
    assert lo < tokens * hidden // per_tile <= hi
    return tokens, hidden


def random_parts(tokens, hidden, block, nparts, seed):
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(nparts):
        q = rng.integers(0, 256, size=(tokens, hidden), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] ^= 0x01                      # no E4M3 NaN codes
        alpha = rng.uniform(0.25, 4.0, size=tokens * hidden // block).astype(np.float32)
        scale = np.float32(rng.uniform(0.5, 50.0))
        parts.append((torch.from_numpy(q).cuda(), torch.from_numpy(alpha).cuda(),
                      torch.tensor([scale], dtype=torch.float32).cuda()))
    return parts


CONFIGS = [(b, t, w) for b, order in ORDER.items() for t, w in order]


@pytest.mark.parametrize("block,tpw,waves", CONFIGS)
@pytest.mark.parametrize("nparts", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fused_decompress_sum_compress_every_variant(taco, block, tpw, waves, nparts):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tokens, hidden = shape_for(block, tpw, waves, cus)
    print(f"[case] fused dsc block={block} tiles/wavefront={tpw} wavefronts={waves} parts={nparts} "
          f"shape=({tokens},{hidden})", flush=True)
    parts = random_parts(tokens, hidden, block, nparts, seed=1000 * block + 100 * waves + 10 * tpw + nparts)
    lib = taco.load()
    ws = torch.zeros(lib.taco_decompress_sum_compress_workspace_bytes(tokens, hidden, block),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > COMPRESS_WORKSPACE
    got = [t.clone() for t in taco.decompress_sum_compress(parts, block, 0.75, workspace=ws)]
    torch.cuda.synchronize()
    assert not taco.workspace_timed_out(ws)
    assert int(torch.count_nonzero(ws[COMPRESS_WORKSPACE:])) == 0, "the two-kernel path ran"
    ref = taco.decompress_sum_compress(parts, block, 0.75, single_pass=False)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


# ------------------------------------------------------------ persistent decompress
# The decompress grid holds at most a few workgroups per CU and each
# wavefront walks its tiles in a loop unrolled by two.  These shapes give
# every wavefront three or four tiles (both halves of the loop, and an odd
# count for some) and end in a partial tile (9 blocks per row, an odd row
# count), checked against the oracle on sampled rows: the first and last
# tiles of the tensor and rows spread over it.
DECOMPRESS_LOOP = {64: (576, 38229), 128: (1152, 51029), 256: (2304, 25779)}


def sample_rows(T, n=96, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(0, 8)) | set(range(T - 8, T)) | set(int(r) for r in rng.integers(0, T, n))
    return np.array(sorted(rows))


@pytest.mark.parametrize("per_block", [False, True])
@pytest.mark.parametrize("block", [64, 128, 256])
def test_decompress_several_tiles_per_wavefront(taco, block, per_block):
    import oracle
    import parity
    hidden, tokens = DECOMPRESS_LOOP[block]
    nblocks = tokens * hidden // block
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = cus * {64: 6, 128: 8, 256: 4}[block] * 4   # at most this many in the grid
    assert -(-nblocks // 16) > 2.5 * waves and nblocks % 16 != 0
    print(f"[case] decompress block={block} per_block={per_block} shape=({tokens},{hidden})", flush=True)
    rng = np.random.default_rng(block + per_block)
    q = rng.integers(0, 256, size=(tokens, hidden), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] ^= 0x01
    alpha = rng.uniform(0.25, 4.0, size=nblocks).astype(np.float32)
    if per_block:
        s = rng.uniform(0.5, 50.0, size=nblocks).astype(np.float32)
        got = taco.decompress_blockscale(torch.from_numpy(q).cuda(), torch.from_numpy(alpha).cuda(),
                                         torch.from_numpy(s).cuda(), block)
    else:
        s = np.float32(rng.uniform(0.5, 50.0))
        got = taco.decompress(torch.from_numpy(q).cuda(), torch.from_numpy(alpha).cuda(),
                              torch.tensor([s], dtype=torch.float32).cuda(), block)
    got = W.bf16_bits(got)
    rows = sample_rows(tokens, seed=block)
    per_row = hidden // block
    blk = (rows[:, None] * per_row + np.arange(per_row)[None, :]).reshape(-1)
    qs, a_s = q[rows], alpha[blk]
    if per_block:
        ref = oracle.decompress_blockscale(qs, a_s, s[blk], block)
        exact = oracle.decompress_blockscale_f64(qs, a_s, s[blk], block)
        bound = parity.decompress_error_bound(qs, a_s, s[blk], block)
    else:
        ref = oracle.decompress(qs, a_s, s, block)
        exact = oracle.decompress_f64(qs, a_s, s, block)
        bound = parity.decompress_error_bound(qs, a_s, s, block)
    parity.bf16_neighbours_ok(got[rows], ref, exact, bound, 1e-4)
