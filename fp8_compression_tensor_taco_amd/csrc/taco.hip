// libtaco: TACO's FP8 compression operator for tensor-parallel intermediate
// tensors, hand-written for AMD Instinct MI355X (gfx950, CDNA4, wave64).
//
// Sources: "TACO pt-summary" = the Portuguese structured summary on gist.science
// of "TACO: Efficient Communication Compression of Intermediate Tensors for
// Scalable Tensor-Parallel LLM Training"; "TACO zh-news" = the Chinese
// euno.news summary of the same paper.  The operator: per-block raw second
// moment and ASH rescale to a target energy, orthonormal Hadamard rotation
// [pt-summary 2.B.1], a post-rotation scale that fits the FP8 range
// [pt-summary 2.B.2; per tensor as in zh-news, method section], E4M3 cast
// [pt-summary 2.A], the inverse [pt-summary 2.B.2], and the local reduction of
// the two-shot all-reduce [pt-summary 2.B.3].
//
// Tiles.  A wavefront works on tiles of 16 consecutive blocks.  Global
// accesses cover whole 64-byte segments or more: bf16 x is copied into LDS
// lane-linearly (1 KiB per instruction) by the fused compress where its tiles
// fit, and read in the MFMA layout (64 contiguous bytes per block per
// instruction) elsewhere; FP8 codes are read
// in the wide layout (one 16-byte load per lane, 64 contiguous bytes per
// quad); compression codes and decompression outputs are staged through a
// padded per-wavefront LDS tile and stored lane-linearly (1 KiB per
// instruction); decompress-sum outputs leave from registers after an
// exchange inside the quad (64 contiguous bytes per quad).
//
// Two compute layouts are used for the Walsh-Hadamard rotation of a block:
//
// * Wide layout (vector ALUs, everything that rotates codes).  Four
//   consecutive lanes (a quad) own one block; within each 64-element group g,
//   lane q holds the 16 consecutive elements 64*g + 16*q + (0..15) as two
//   8-element chunks.  Butterflies on the element-index bits a lane holds
//   (0-3 and 6..) are in-lane; bits 4 and 5 cross lanes inside the quad,
//   where a DPP quad permutation reaches the partner.  That butterfly is
//   computed as v + c*partner with a per-lane sign c = +-1; lanes whose index
//   bit is set then hold the negation of their output.  The negation is
//   tracked, not undone: after both quad stages lane q holds its outputs
//   times D(q) = c1(q)*c2(q), and D is folded into the scale applied next.
//
// * MFMA layout (matrix cores, compression).  The rotation of raw x is the
//   dense product y = H_B x with a +-1 matrix, and x is exactly bf16, so
//   v_mfma_f32_16x16x32_bf16 computes it with exact products and fp32 sums.
//   See the MFMA section below.
//
// Compression needs the tensor-wide max|y| before any code can be written.
// When the tensor fits in the registers of the resident wavefronts (its
// rotated blocks, or for larger tensors its bf16 input) it is one kernel with
// a grid-wide barrier (see the fused section); otherwise two kernels over the
// same tiles: a statistics pass (energy, alpha, rotation, per-workgroup max)
// and a quantisation pass that folds the workgroup maxima into s, re-reads x
// and writes the codes.  An INT8 absmax path (no rotation) sits at the end.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cstddef>
#include <initializer_list>
#include <mutex>
#include <utility>

#include "taco.h"

namespace {

constexpr int kTileBlocks = 16;         // blocks per wavefront tile
constexpr int kThreads = 256;           // decompress workgroups: 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kThreadsC = 1024;         // compress workgroups: 16 wavefronts
constexpr int kWavesC = kThreadsC / 64;
constexpr float kQmax = 448.0f;         // largest E4M3FN magnitude
constexpr float kMinEnergy = 0x1p-40f;  // accepted target energies
constexpr float kMaxEnergy = 0x1p40f;
constexpr int kMaxPartials = 1024;      // workgroups of the statistics pass (at most)

constexpr int kQuadXor1 = 0xB1;         // DPP quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;         // DPP quad_perm [2,3,0,1]

template <int B>
struct Blk {
  static constexpr int NA = B / 32;               // 8-element chunks per lane of a quad
  static constexpr int C16 = B / 8;               // 16-byte bf16 chunks per block
  static constexpr float inv_b = 1.0f / B;        // exact (power of two)
  static constexpr float rsqrt_b = B == 64 ? 0.125f
                                 : B == 128 ? 0.0883883476483184405f  // fp32(1/sqrt(128))
                                            : 0.0625f;
  // LDS tile row stride (bytes) of codes in the MFMA layout; the padding makes
  // the compute-layout writes conflict-free (16 lanes hit 16 bank groups).
  static constexpr int kCodeRowMfma = B + 16;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- helpers

// Streaming accesses.  Non-temporal stores of the outputs leave no dirty
// lines in L2 for the end-of-kernel write-back (measured: compress 17.2 ->
// 15.0 us, decompress 13.7 -> 12.1 us per call on [4096, 4096]; the
// decompress-sum output gains only together with its 16-byte code loads:
// 22.5 -> 20.1 us for 4 parts).
// x is read non-temporally by the fused kernel (14.9 -> 14.2 us), but not by
// the two-pass kernels (the quantisation pass reads the statistics pass's
// data again from the cache; non-temporal loads there measured slower).
// Non-temporal code loads measured slower too (decompress 12.0 -> 15.8 us).
#ifndef TACO_NT_Q_LOADS
#define TACO_NT_Q_LOADS 0
#endif
#ifndef TACO_NT_CODE_STORES
#define TACO_NT_CODE_STORES 1
#endif
#ifndef TACO_NT_OUT_STORES
#define TACO_NT_OUT_STORES 1
#endif
// The fused compress stages x through LDS where its tiles fit (see
// compress_fused_lds_kernel); 0 selects the direct MFMA-layout loads.
#ifndef TACO_FUSED_LDS
#define TACO_FUSED_LDS 1
#endif
#ifndef TACO_NT_SUM_STORES
#define TACO_NT_SUM_STORES 1
#endif
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ void store16(uint4* p, const uint4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), reinterpret_cast<u32x4_t*>(p));
  else
    *p = v;
}

template <bool NT>
__device__ __forceinline__ void store8(uint2* p, const uint2 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2_t, v), reinterpret_cast<u32x2_t*>(p));
  else
    *p = v;
}

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT)
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  else
    return *p;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float dot2_bf16(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum of squares of NC chunks of 8 bf16 values: exact products, accumulated
// in fp32 by v_dot2c chains (two or four independent chains, then added), so
// the relative rounding error stays below (B/8 + 2) * 2^-24.
template <int NC>
__device__ __forceinline__ float sum_squares_bf16(const uint4 (&u)[NC]) {
  constexpr int kChains = NC >= 4 ? 4 : 2;
  float acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = 0.0f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float& a = acc[i % kChains];
    a = dot2_bf16(u[i].x, u[i].x, a);
    a = dot2_bf16(u[i].y, u[i].y, a);
    a = dot2_bf16(u[i].z, u[i].z, a);
    a = dot2_bf16(u[i].w, u[i].w, a);
  }
  float ss = acc[0];
#pragma unroll
  for (int c = 1; c < kChains; ++c) ss += acc[c];
  return ss;
}

// Butterflies on index bits [lo, 3) inside one 8-value chunk.
template <int LO>
__device__ __forceinline__ void fwht_chunk(float (&v)[8]) {
#pragma unroll
  for (int h = LO; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
}

// v[j] <- v[j] + dpp<CTRL>(v[j]) * c for the 8 values of a chunk, each in one
// vector instruction: the quad permutation applied as a DPP modifier to the
// first source of v_fmac_f32 (for fmaf(dpp<CTRL>(v), c, v) the compiler
// emits a v_mov_b32_dpp and a v_fmac_f32, twice the vector instructions).
// The same single rounding, so the same results.  A DPP source must not have
// been written by a vector instruction in the two cycles before it is read,
// and the compiler does not look inside inline assembly for that hazard:
// an s_nop of two wait states on each side covers it.
template <int CTRL>
__device__ __forceinline__ void fmac_dpp8(float (&v)[8], float c) {
  static_assert(CTRL == kQuadXor1 || CTRL == kQuadXor2, "quad permutations only");
#define TACO_FMAC_DPP(i, perm) "v_fmac_f32_dpp %" #i ", %" #i ", %8 quad_perm:" perm \
                               " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define TACO_FMAC_DPP8(perm)                                                                  \
  asm("s_nop 1\n\t" TACO_FMAC_DPP(0, perm) TACO_FMAC_DPP(1, perm) TACO_FMAC_DPP(2, perm)         \
      TACO_FMAC_DPP(3, perm) TACO_FMAC_DPP(4, perm) TACO_FMAC_DPP(5, perm) TACO_FMAC_DPP(6, perm) \
      TACO_FMAC_DPP(7, perm) "s_nop 1"                                                         \
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),     \
        "+v"(v[7])                                                                            \
      : "v"(c))
  if constexpr (CTRL == kQuadXor1)
    TACO_FMAC_DPP8("[1,0,3,2]");
  else
    TACO_FMAC_DPP8("[2,3,0,1]");
#undef TACO_FMAC_DPP8
#undef TACO_FMAC_DPP
}

// One butterfly stage on an index bit held across the quad (CTRL: the DPP
// quad permutation that pairs the lanes differing in it), with its sign debt
// c: v <- v + c * (the partner lane's v).  FUSED folds the exchange into the
// multiply-add (fmac_dpp8); otherwise the compiler moves the partner's value
// first (v_mov_b32_dpp, then v_fmac_f32).  Both round once: the results are
// identical.
template <int NA, int CTRL, bool FUSED = false>
__device__ __forceinline__ void fwht_quad_stage(float (&v)[NA][8], float c) {
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    if constexpr (FUSED) {
      fmac_dpp8<CTRL>(v[a], c);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[a][j] = fmaf(dpp<CTRL>(v[a][j]), c, v[a][j]);
    }
  }
}

// One butterfly stage on the index bit that selects chunk c or c + H.
template <int NA, int H>
__device__ __forceinline__ void fwht_chunk_stage(float (&v)[NA][8]) {
#pragma unroll
  for (int a = 0; a < NA; a += 2 * H)
#pragma unroll
    for (int c = a; c < a + H; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = v[c][j], y = v[c + H][j];
        v[c][j] = x + y;
        v[c + H][j] = x - y;
      }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Max over a workgroup of WAVES wavefronts; every thread gets the result.
template <int WAVES>
__device__ __forceinline__ float workgroup_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) m = fmaxf(m, red[w]);
  return m;
}

// ASH scale from the block's sum of squares ss = B * m:
//   alpha = sqrt(E / m) = sqrt(E * B) * rsqrt(ss),  1 if the block is zero.
// sqrt_eb = fp32(sqrt(E * B)) is computed once on the host; v_rsq_f32 is
// accurate to 1 ulp, so alpha is within a few ulps of the correctly rounded
// value.  Both compress passes evaluate it identically.
__device__ __forceinline__ float ash_scale(float ss, float sqrt_eb) {
  return ss > 0.0f ? sqrt_eb * __builtin_amdgcn_rsqf(ss) : 1.0f;
}

// 8 E4M3FN codes -> fp32 (exact).
__device__ __forceinline__ void from_fp8x8(const uint2 u, float (&v)[8]) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(u.x), false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(u.x), true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(u.y), false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(u.y), true);
  v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  v[4] = c[0]; v[5] = c[1]; v[6] = d[0]; v[7] = d[1];
}

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const bf16x2_t r = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(unsigned, r);
}

__device__ __forceinline__ uint4 to_bf16x8(const float (&v)[8], float c) {
  return make_uint4(pack_bf16x2(v[0] * c, v[1] * c), pack_bf16x2(v[2] * c, v[3] * c),
                    pack_bf16x2(v[4] * c, v[5] * c), pack_bf16x2(v[6] * c, v[7] * c));
}

// Lane-linear transfer of a tile between global memory and its padded LDS
// image: tile row r (block 16t + r) holds ROW bytes, stored at r * STRIDE.
// Only rows of blocks that exist are transferred.
template <int ROW, int STRIDE, bool NT>
__device__ __forceinline__ void lds_store_tile_to_global(const char* lds, uint4* __restrict__ g,
                                                         int64_t tile, int rows_valid) {
  constexpr int kChunksPerRow = ROW / 16, kChunks = kTileBlocks * kChunksPerRow;
  const int lane = threadIdx.x & 63;
  uint4* base = g + tile * kChunks;
  if (rows_valid == kTileBlocks && kChunks % 64 == 0) {      // whole tile: no lane predicates
#pragma unroll
    for (int i = 0; i < kChunks / 64; ++i) {
      const int c = 64 * i + lane;
      store16<NT>(&base[c], *reinterpret_cast<const uint4*>(lds + (c / kChunksPerRow) * STRIDE + 16 * (c % kChunksPerRow)));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < (kChunks + 63) / 64; ++i) {
    const int c = 64 * i + lane;
    const int r = c / kChunksPerRow, col = c % kChunksPerRow;
    if (c < kChunks && r < rows_valid)
      store16<NT>(&base[c], *reinterpret_cast<const uint4*>(lds + r * STRIDE + 16 * col));
  }
}

// The wavefront's index in its workgroup, as a wave-uniform (scalar) value:
// the compiler cannot tell that threadIdx.x / 64 is uniform, and would
// otherwise keep every tile index derived from it in a pair of VGPRs per lane.
__device__ __forceinline__ int wave_in_group() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// A wave-uniform 64-bit value moved to SGPRs.  The builtin returns int, so
// each half goes through unsigned before it is widened: widening the int
// itself would sign-extend the low half into the high one.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<unsigned>(v))));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<unsigned>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ int rows_valid(int64_t tile, int64_t nblocks) {
  const int64_t r = nblocks - tile * kTileBlocks;
  return r >= kTileBlocks ? kTileBlocks : static_cast<int>(r);
}

// Lane geometry of a quad (the four lanes that own one block of a 16-block tile).
struct Quad {
  int blk;        // block of the tile owned by this lane's quad (0..15)
  int ql;         // position in the quad (0..3)
  float c1, c2;   // butterfly signs of the two quad stages
  float debt;     // c1*c2: sign the quad stages leave on this lane's outputs
  __device__ __forceinline__ Quad() {
    const int lane = threadIdx.x & 63;
    blk = lane >> 2;
    ql = lane & 3;
    c1 = (ql & 1) ? -1.0f : 1.0f;
    c2 = (ql & 2) ? -1.0f : 1.0f;
    debt = c1 * c2;
  }
};

// ============================================================== MFMA engine
//
// The product is formed transposed, C[m][n] = sum_k H[m][k] X[n][k], with the
// 16 columns n of the MFMA being the 16 blocks of a tile:
//   B operand: lane (g, n), g = lane/16, holds 8 elements of block n,
//              element 32*kt + 8*g + s (s = 0..7) in K-step kt;
//   A operand: lane (g, r) holds H[16*mt + r][32*kt + 8*g + s];
//   C:         lane (g, n) receives y[block n][16*mt + 4*g + i], i = 0..3.
// Because H[i][j] = (-1)^popcount(i & j) factors over index bits, the A
// operand for M-tile mt and K-step kt is F_{mt&1} * (-1)^popcount((mt>>1) & kt)
// with two lane-dependent fragments
//   F_e[lane (g, r)][s] = (-1)^(popcount(r & s & 7) + (r>>3)*(g&1) + e*(g>>1)),
// so four constant register sets (F_0, F_1 and their negations) cover every
// (mt, kt) pair.  The B operand is read straight from global memory: for each
// block the four lanes g of its column read 64 contiguous bytes.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct HadFrag {
  bf16x8_t pos[2];   // F_0, F_1
  bf16x8_t neg[2];   // -F_0, -F_1
};

__device__ __forceinline__ HadFrag make_hadamard_fragments() {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  HadFrag F;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    unsigned short bits[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int par = __builtin_popcount(r & s & 7) + ((r >> 3) & g & 1) + (e & (g >> 1));
      bits[s] = (par & 1) ? 0xBF80 : 0x3F80;   // bf16 -1.0 / +1.0
    }
    uint4 u = make_uint4(bits[0] | (unsigned(bits[1]) << 16), bits[2] | (unsigned(bits[3]) << 16),
                         bits[4] | (unsigned(bits[5]) << 16), bits[6] | (unsigned(bits[7]) << 16));
    F.pos[e] = __builtin_bit_cast(bf16x8_t, u);
    u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
    F.neg[e] = __builtin_bit_cast(bf16x8_t, u);
  }
  return F;
}

// Rows 16*mt .. 16*mt+15 of H_B applied to the 16 blocks of the tile.
template <int B>
__device__ __forceinline__ f32x4_t hadamard_mtile(const HadFrag& F, const uint4 (&xr)[B / 32], int mt) {
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kt = 0; kt < B / 32; ++kt) {
    const bool neg = __builtin_popcount((mt >> 1) & kt) & 1;
    const bf16x8_t a = neg ? F.neg[mt & 1] : F.pos[mt & 1];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, xr[kt]), acc, 0, 0, 0);
  }
  return acc;
}

// Sum of squares of a column's block: the lane's B/4 elements, then the 4
// lanes g = 0..3 of the column (lanes n, n+16, n+32, n+48), combined with the
// gfx950 row swaps: permlane32_swap pairs lane l with l^32 and permlane16_swap
// pairs l with l^16.  Each step adds the same two operands in the same order
// in both lanes of a pair, so every lane of the column gets the same sum.
__device__ __forceinline__ float column_sum_rows(float ss) {
  const unsigned u = __float_as_uint(ss);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  ss = __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
  const unsigned v = __float_as_uint(ss);
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
}

template <int B>
__device__ __forceinline__ float column_sum_squares(const uint4 (&xr)[B / 32]) {
  return column_sum_rows(sum_squares_bf16<B / 32>(xr));
}

// The B operand of one tile.  Loads are branch-free: lanes whose block lies
// past the end of the tensor read the tile's last block instead, and their
// results are never stored (or are duplicates of a valid column's).
template <int B, bool NT>
__device__ __forceinline__ void load_tile_mfma(const uint4* __restrict__ x, int64_t t, int64_t nblocks,
                                               uint4 (&xr)[B / 32]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int rv = rows_valid(t, nblocks);
  const uint4* tile = x + t * (kTileBlocks * Blk<B>::C16);
  const int row = n < rv ? n : rv - 1;
#pragma unroll
  for (int kt = 0; kt < B / 32; ++kt) xr[kt] = load16<NT>(&tile[row * Blk<B>::C16 + 4 * kt + g]);
}

// Codes of rows 16 mt .. 16 mt + 15 of a tile's rotated blocks (MFMA C
// layout): scale by c, convert, and place them in the wavefront's LDS tile.
template <int B>
__device__ __forceinline__ void codes_to_lds_mfma(const f32x4_t y, float c, int mt, char* lds) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  int wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] * c, y[1] * c, 0, false);
  wd = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] * c, y[3] * c, wd, true);
  *reinterpret_cast<int*>(lds + n * Blk<B>::kCodeRowMfma + 16 * mt + 4 * g) = wd;
}

// ============================================================== LDS staging of x
//
// The compress kernels stage x through LDS: each wavefront copies its tiles
// into its own LDS region with global_load_lds_dwordx4 (16 bytes per lane
// written straight to LDS at lane-linear positions, 1 KiB per instruction),
// so every load instruction covers whole cache lines instead of the 64-byte
// pieces of loads in the MFMA operand layout; the B operand is then read
// from LDS.  Which global chunk a lane fetches is free as long as each
// instruction covers its 1 KiB, so chunk k of block n is fetched by the lane
// that writes position k ^ swz(n) of the block's LDS row: the 16 columns of
// one K-step then read 16 different 16-byte bank groups.
template <int B>
struct LdsTile {
  static constexpr int C16 = B / 8;                        // 16-byte chunks per block
  static constexpr int kBytes = kTileBlocks * B * 2;       // one bf16 tile
  static constexpr int kCopies = kBytes / 1024;            // copy instructions per tile
  // B = 64: a 256-byte LDS row holds two blocks, so the low bit of n picks
  // the half and the swizzle uses the next three; otherwise the low four.
  static __device__ __forceinline__ int swz(int n) { return B == 64 ? (n >> 1) & 7 : n & 15; }
};

// One gfx950 direct-to-LDS copy: lane i writes the 16 bytes at base + off
// (base wave-uniform, in an SGPR pair; off a per-lane byte offset) to LDS
// address lds + 16 i (lds is wave-uniform, in m0), non-temporal like the
// direct loads.  Written as inline asm because with the compiler's builtin it
// waits for every copy in flight before the wavefront's first LDS read
// (vmcnt(0)), which serialises each tile's rotation behind all of the
// wavefront's copies; the caller waits instead with wait_copies, tile by
// tile.  One wait state separates the write of m0 from the copy that reads
// it.  No VGPR is written, and the offset VGPR is read at issue.  Nothing
// else in these kernels uses m0.
// (clang warns that m0 is a reserved register and its clobber may not be
// honoured; the compiler uses m0 nowhere in this file on gfx950, which
// tests/test_build_checks.py checks on the generated assembly.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const uint4* base, unsigned off, unsigned lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

// Waits until at most N vector memory operations of the wavefront are in
// flight.  Loads complete in issue order, so after the copies of tiles
// 0..i and then of N / kCopies more tiles, wait_copies<N> means tiles 0..i
// have landed (earlier operations, such as the barrier's leaf add and load,
// only make it wait longer).  The memory clobber keeps the LDS reads after it;
// the scheduling barrier keeps the previous tile's matrix and vector work
// before it (the scheduler would otherwise sink some of it below the wait).
template <int N>
__device__ __forceinline__ void wait_copies() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Copies tile t (clamped by the caller) into lds_tile; blocks past the end of
// the tensor are filled with the tile's last block, as load_tile_mfma does.
template <int B>
__device__ __forceinline__ void copy_tile_to_lds(const uint4* __restrict__ x, int64_t t, int64_t nblocks,
                                                 char* lds_tile) {
  constexpr int C16 = LdsTile<B>::C16;
  const int lane = threadIdx.x & 63;
  const int rv = rows_valid(t, nblocks);
  // t is wave-uniform, so the tile's address goes to SGPRs and each copy
  // needs one offset VGPR (the same for every whole tile)
  const uint4* tile = reinterpret_cast<const uint4*>(uniform_u64(reinterpret_cast<uint64_t>(x + t * (kTileBlocks * C16))));
  const unsigned base = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds_tile)));
#pragma unroll
  for (int d = 0; d < LdsTile<B>::kCopies; ++d) {
    const int pos = 64 * d + lane;
    const int n = pos / C16, p = pos % C16;
    const int row = n < rv ? n : rv - 1;
    copy16_to_lds(tile, 16u * static_cast<unsigned>(row * C16 + (p ^ LdsTile<B>::swz(n))), base + 1024 * d);
  }
}

template <int B>
__device__ __forceinline__ void read_tile_from_lds(const char* lds_tile, uint4 (&xr)[B / 32]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
#pragma unroll
  for (int kt = 0; kt < B / 32; ++kt)
    xr[kt] = *reinterpret_cast<const uint4*>(
        lds_tile + 16 * (n * LdsTile<B>::C16 + ((4 * kt + g) ^ LdsTile<B>::swz(n))));
}

// Waits until this wavefront's LDS reads have returned (before a copy may
// overwrite the region they read).
__device__ __forceinline__ void lds_reads_done() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// Two-pass compression, for tensors whose rotated blocks do not fit in the
// resident wavefronts' registers (or when the single pass is switched off):
// a statistics kernel (alpha and per-workgroup max) and a quantisation kernel
// that folds the workgroup maxima into s, re-reads x and writes the codes.
// Both give each wavefront U tiles per trip (wid, wid + W, ... for W
// wavefronts in the grid), issue all of a trip's loads before using any, and
// keep every branch away from loads in flight (the compiler waits for all
// outstanding loads at a join).  Tiles past the end load, and write alpha
// for, the last tile again (identical values).  The arithmetic per tile is
// the fused kernel's, instruction for instruction, so the results are
// bitwise identical.
template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_stats_mfma_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb,
    float* __restrict__ alpha, float* __restrict__ partial) {
  constexpr int NK = B / 32, NM = B / 16;
  __shared__ float red[kWaves];
  const HadFrag F = make_hadamard_fragments();
  const int n = threadIdx.x & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWaves;
  float amax = 0.0f;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + wave_in_group(); t0 < ntiles;
       t0 += nw * U) {
    uint4 xr[U][NK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u * nw;
      load_tile_mfma<B, false>(x, t < ntiles ? t : ntiles - 1, nblocks, xr[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u * nw;
      const int64_t tc = t < ntiles ? t : ntiles - 1;
      const int rv = rows_valid(tc, nblocks);
      const float al = ash_scale(column_sum_squares<B>(xr[u]), sqrt_eb);
      alpha[tc * kTileBlocks + (n < rv ? n : rv - 1)] = al;
      float m = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const f32x4_t v = hadamard_mtile<B>(F, xr[u], mt);
        m = fmaxf(fmaxf(m, fabsf(v[0])), fabsf(v[1]));
        m = fmaxf(fmaxf(m, fabsf(v[2])), fabsf(v[3]));
      }
      if (t < ntiles && n < rv) amax = fmaxf(amax, m * (al * Blk<B>::rsqrt_b));
    }
  }
  const float wg = workgroup_max<kWaves>(amax, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = wg;
}

// Max of the n (<= kMaxPartials) workgroup maxima; every thread of the
// workgroup takes part (kMaxPartials / kThreads loads each, issued together,
// indices clamped so that no branch surrounds them) and gets the result.
__device__ __forceinline__ float partials_max(const float* __restrict__ partial, int n, float* red) {
  constexpr int kPer = kMaxPartials / kThreads;
  float v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = static_cast<int>(threadIdx.x) + kThreads * k;
    v[k] = partial[i < n ? i : n - 1];
  }
  float m = v[0];
#pragma unroll
  for (int k = 1; k < kPer; ++k) m = fmaxf(m, v[k]);
  return workgroup_max<kWaves>(m, red);
}

template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_quant_mfma_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb,
    const float* __restrict__ partial, int npartial, float* __restrict__ scale,
    uint4* __restrict__ q) {
  constexpr int NK = B / 32, NM = B / 16, SROW = Blk<B>::kCodeRowMfma;
  __shared__ float red[kWaves];
  __shared__ __attribute__((aligned(16))) char lds_all[kWaves][kTileBlocks * SROW];
  char* lds = lds_all[threadIdx.x >> 6];
  const HadFrag F = make_hadamard_fragments();
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + wave_in_group();
  uint4 xr[U][NK];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + u * nw;
    load_tile_mfma<B, false>(x, t < ntiles ? t : ntiles - 1, nblocks, xr[u]);
  }
  const float A = partials_max(partial, npartial, red);
  const float s = A == 0.0f ? 1.0f : kQmax / A;   // NaN stays NaN
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t t = t0 + u * nw;
    if (t >= ntiles) break;
    const float c = (ash_scale(column_sum_squares<B>(xr[u]), sqrt_eb) * s) * Blk<B>::rsqrt_b;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(hadamard_mtile<B>(F, xr[u], mt), c, mt, lds);
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(lds, q, t, rows_valid(t, nblocks));
    __builtin_amdgcn_wave_barrier();
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
}

// ============================================================== fused compress
//
// One kernel for the whole compression when the tensor fits on chip.  Every
// wavefront loads its TPW tiles of raw bf16 x, computes alpha and the rotated
// blocks y = H x on the matrix cores, keeps y (HOLD_Y) or x (otherwise) in
// VGPRs, and contributes to a grid-wide max of alpha |y| / sqrt(B).  After a
// grid-wide barrier that yields that max, it scales, converts and stores its
// codes straight from registers (recomputing y from x when only x is held).
// x is read from HBM once and the codes are written once, the single fused
// pass the pages describe [TACO pt-summary, 2.B.3].
//
// Grid barrier.  The launch makes every workgroup resident at once (grid <=
// occupancy x CUs, and at most one workgroup per CU).  The only value
// exchanged is the max, so the barrier is built from device-scope atomic
// loads, stores and adds alone, with no fences
// (a device-scope release or acquire would write back or invalidate the whole
// L2).  Two parts:
//  * Call number.  Leaf lines of kLeafWgs workgroups each hold a running
//    64-bit count that never resets and advances by exactly kLeafWgs per
//    call: every workgroup adds 1 to its leaf (the first of a partial leaf
//    also adds the missing arrivals) and workgroup 0 adds kLeafWgs to every
//    leaf the grid does not use.  A workgroup's own add therefore returns a
//    value that tells it the call number c, without reading any state first.
//    It is issued while the workgroup's input loads are in flight, so it is
//    off the critical path.
//  * Exchange.  Each workgroup stores (c + 1) << 32 | max bits into its own
//    slot (one 64-bit store; non-negative floats order like their bits), then
//    wavefront 0 polls the slots of the whole grid until all of them carry
//    epoch c + 1 and takes their max.  After the last arrival only that store
//    and one round of polls remain (the previous protocol's chain of leaf and
//    root atomics took about 1 us longer per call).  Slots of workgroups
//    beyond this grid are never read; a slot can only hold epoch c + 1 if it
//    was written in this call, since epochs only grow (zero-filling the
//    workspace resets counts and slots together).
// Epochs are the low 32 bits of the call number, and a slot left from long
// ago could carry the current epoch after 2^32 calls.  So workgroup 0 also
// writes the current epoch into every slot beyond this grid: after any call
// every one of the kMaxSlots slots holds that call's epoch, and the next call
// waits for the next epoch, which differs from it whatever the grid sizes.
// The poll is bounded (spin_limit polls, chosen per call by the host): a
// workgroup that gives up sets the sticky timed_out flag and takes NaN as the
// max, so its codes are all E4M3 NaN rather than plausible values under a
// stale scale.  It has already counted itself and stored its slot, so the
// barrier still completes for the others and the workspace stays consistent
// for the next call; every wavefront finishes.

constexpr int kLine = 256;               // bytes per leaf line
constexpr int kLeafWgs = 16;             // workgroups per leaf
constexpr int kLeaves = 64;              // leaf lines => at most 1024 fused workgroups
constexpr size_t kPartialOffset = static_cast<size_t>(kLine) * (1 + kLeaves);
constexpr size_t kSlotOffset = kPartialOffset + kMaxPartials * sizeof(float);
constexpr int kSlotStride = 16;          // bytes per workgroup slot
constexpr int kMaxSlots = kLeaves * kLeafWgs;
constexpr unsigned kDefaultSpinLimit = TACO_DEFAULT_BARRIER_POLLS;

struct RootLine {
  unsigned long long unused;
  unsigned timed_out;
};

struct LeafLine {
  unsigned long long count;
};

__device__ __forceinline__ LeafLine* leaf_line(char* ws, unsigned l) {
  return reinterpret_cast<LeafLine*>(ws + kLine * (1 + l));
}

__device__ __forceinline__ unsigned long long* slot_of(char* ws, unsigned wg) {
  return reinterpret_cast<unsigned long long*>(ws + kSlotOffset + static_cast<size_t>(kSlotStride) * wg);
}

template <typename T>
__device__ __forceinline__ T load_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void store_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ T add_agent(T* p, T v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts this workgroup into its leaf; called by the 64 lanes of wavefront 0
// (lane 0 adds this workgroup's arrivals; in workgroup 0, lane l >= the grid's
// leaf count advances leaf l).  The adds return nothing; later every lane of
// wavefront 0 loads its workgroup's leaf count (leaf_count), with no branch
// around the load, so that nothing waits for it before the barrier needs it.
// That count lies in [16 c + 1, 16 c + 16] for call number c: this
// workgroup's own add precedes the load in wavefront 0's program order on the
// same word, every leaf stood at 16 c when the call began, and the call adds
// exactly 16.
__device__ __forceinline__ void arrive_add_wave0(char* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const unsigned l = blockIdx.x / kLeafWgs;
  const unsigned nleaves = (gridDim.x + kLeafWgs - 1) / kLeafWgs;
  if (lane == 0) {
    const unsigned in_leaf = min(static_cast<unsigned>(kLeafWgs), gridDim.x - l * kLeafWgs);
    unsigned long long inc = 1;
    if (blockIdx.x % kLeafWgs == 0) inc += kLeafWgs - in_leaf;
    add_agent(&leaf_line(ws, l)->count, inc);
  } else if (blockIdx.x == 0 && static_cast<unsigned>(lane) >= nleaves) {
    add_agent(&leaf_line(ws, lane)->count, static_cast<unsigned long long>(kLeafWgs));
  }
}
static_assert(kLeaves == 64, "arrive_add_wave0 advances one unused leaf per lane");

// This workgroup's leaf count (other wavefronts may load it too, but only
// wavefront 0's load is ordered after the workgroup's own add).
__device__ __forceinline__ unsigned long long leaf_count(char* __restrict__ ws) {
  return load_agent(&leaf_line(ws, blockIdx.x / kLeafWgs)->count);
}

__device__ __forceinline__ unsigned long long arrive_wave0(char* __restrict__ ws) {
  arrive_add_wave0(ws);
  return leaf_count(ws);
}

// One round of polls for grids of at most 256 workgroups: this lane's 4
// slots (slot 0, which this call writes too, stands in past the grid).
__device__ __forceinline__ void poll_round(char* __restrict__ ws, unsigned lane, unsigned long long (&r)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const unsigned j = lane + 64 * k;
    r[k] = load_agent(slot_of(ws, j < gridDim.x ? j : 0));
  }
}

// Whether every slot of a round carries the epoch; m gets the round's max.
__device__ __forceinline__ bool round_ready(const unsigned long long (&r)[4], unsigned epoch, unsigned& m) {
  bool ok = true;
  unsigned mm = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ok = ok && static_cast<unsigned>(r[k] >> 32) == epoch;
    mm = max(mm, static_cast<unsigned>(r[k]));
  }
  m = mm;
  return __builtin_amdgcn_ballot_w64(!ok) == 0;
}

// Grid-wide max; called by the 64 lanes of wavefront 0 with the workgroup's
// max (uniform) and the leaf count arrive_wave0 returned.  Every lane returns
// the tensor-wide max, or NaN if this workgroup gave up waiting.
//
// Up to 256 workgroups, two rounds of polls are in flight: round k + 1 is
// issued before round k is checked, so a store is seen about half a round
// sooner (a round is a trip to the memory side, about 0.8 us under load).
// A check only accepts values loaded after the previous check began, so the
// protocol is unchanged.  Cold per call: [4096, 1600] at B = 64 8.64 ->
// 8.21 us, [8192, 3584] at B = 128 19.7 -> 19.6 us, [4096, 4096] at B = 128
// unchanged.
__device__ float grid_max_wave0(float wg_max, unsigned long long leaf_count, char* __restrict__ ws,
                                unsigned spin_limit) {
  const int lane = threadIdx.x & 63;
  const unsigned long long v = uniform_u64(leaf_count);
  const unsigned epoch = static_cast<unsigned>((v - 1) / kLeafWgs) + 1;   // call number + 1
  if (lane == 0)
    store_agent(slot_of(ws, blockIdx.x), (static_cast<unsigned long long>(epoch) << 32) | __float_as_uint(wg_max));
  if (blockIdx.x == 0)   // the slots beyond the grid take this call's epoch too
    for (unsigned j = gridDim.x + lane; j < kMaxSlots; j += 64)
      store_agent(slot_of(ws, j), static_cast<unsigned long long>(epoch) << 32);
  unsigned m = 0, spins = 0;
  bool ready = false;
  if (gridDim.x <= 4 * 64) {
    unsigned long long ra[4], rb[4];
    poll_round(ws, lane, ra);
    while (true) {
      poll_round(ws, lane, rb);
      if ((ready = round_ready(ra, epoch, m)) || ++spins >= spin_limit) break;
      poll_round(ws, lane, ra);
      if ((ready = round_ready(rb, epoch, m)) || ++spins >= spin_limit) break;
    }
  } else {
    while (true) {
      bool ok = true;
      unsigned mm = 0;
      for (unsigned j = lane; j < gridDim.x; j += 64) {
        const unsigned long long r = load_agent(slot_of(ws, j));
        ok = ok && static_cast<unsigned>(r >> 32) == epoch;
        mm = max(mm, static_cast<unsigned>(r));
      }
      m = mm;
      if ((ready = __builtin_amdgcn_ballot_w64(!ok) == 0) || ++spins >= spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (!ready) {
    if (lane == 0) store_agent(&reinterpret_cast<RootLine*>(ws)->timed_out, 1u);
    m = 0x7FC00000u;   // quiet NaN: the codes of this workgroup become NaN
  }
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), k)));
  return __uint_as_float(m);
}

// Wavefront w of W owns tiles w, w + W, ..., w + (TPW-1) W (those < ntiles).
// This form loads x straight into the MFMA operand layout; the default build
// launches the LDS-staged kernels below instead (the same arithmetic), and
// this one only where TACO_FUSED_LDS is 0.
template <int B, int TPW, bool HOLD_Y, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void compress_fused_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb, float* __restrict__ alpha,
    float* __restrict__ scale, char* __restrict__ ws, uint4* __restrict__ q, unsigned spin_limit) {
  constexpr int NK = B / 32, NM = B / 16, SROW = Blk<B>::kCodeRowMfma;
  __shared__ float red[WAVES];
  __shared__ float amax_sh;
  __shared__ __attribute__((aligned(16))) char lds_all[WAVES][kTileBlocks * SROW];
  char* lds = lds_all[threadIdx.x >> 6];
  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * WAVES + wave_in_group();
  const int64_t nw = static_cast<int64_t>(gridDim.x) * WAVES;
  // No branch may separate these loads from their first use: the compiler
  // would wait for every outstanding load at the join.  Tiles past the end
  // load (and below store) the last tile again, with identical values.
  uint4 xr[TPW][NK];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    load_tile_mfma<B, true>(x, t < ntiles ? t : ntiles - 1, nblocks, xr[i]);
  }
  // counted into the barrier while the loads are in flight
  unsigned long long leaf = 0;
  if (threadIdx.x < 64) leaf = arrive_wave0(ws);
  f32x4_t y[HOLD_Y ? TPW : 1][NM];
  float al[TPW];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    al[i] = ash_scale(column_sum_squares<B>(xr[i]), sqrt_eb);
    alpha[tc * kTileBlocks + (n < rv ? n : rv - 1)] = al[i];
    float m = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const f32x4_t v = hadamard_mtile<B>(F, xr[i], mt);
      if (HOLD_Y) y[HOLD_Y ? i : 0][mt] = v;
      m = fmaxf(fmaxf(m, fabsf(v[0])), fabsf(v[1]));
      m = fmaxf(fmaxf(m, fabsf(v[2])), fabsf(v[3]));
    }
    if (t < ntiles && n < rv) amax = fmaxf(amax, m * (al[i] * Blk<B>::rsqrt_b));
  }
  const float wg = workgroup_max<WAVES>(amax, red);
  if (threadIdx.x < 64) {
    const float A = grid_max_wave0(wg, leaf, ws, spin_limit);
    if (threadIdx.x == 0) amax_sh = A;
  }
  __syncthreads();
  const float A = amax_sh;
  const float s = A == 0.0f ? 1.0f : kQmax / A;   // NaN stays NaN
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    if (t >= ntiles) continue;
    const float c = (al[i] * s) * Blk<B>::rsqrt_b;
    if (HOLD_Y) {
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(y[HOLD_Y ? i : 0][mt], c, mt, lds);
    } else {
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(hadamard_mtile<B>(F, xr[i], mt), c, mt, lds);
    }
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(lds, q, t, rows_valid(t, nblocks));
    __builtin_amdgcn_wave_barrier();
  }
}

// The same kernel with x staged through LDS (see "LDS staging of x" above),
// for the configurations that hold y: a workgroup's tiles then take at most
// 128 KiB, within gfx950's 160 KiB of LDS per CU (at B = 256 one tile per
// wavefront, 126 VGPRs; [4096, 4096] 14.4 -> 13.9 us against the direct
// loads).  The arithmetic per tile, and so the result, is that of
// compress_fused_kernel.
template <int B, int TPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void compress_fused_lds_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb, float* __restrict__ alpha,
    float* __restrict__ scale, char* __restrict__ ws, uint4* __restrict__ q, unsigned spin_limit) {
  constexpr int NK = B / 32, NM = B / 16, SROW = Blk<B>::kCodeRowMfma, TB = LdsTile<B>::kBytes;
  static_assert(WAVES * TPW * TB <= 128 * 1024, "x tiles exceed the LDS budget");
  static_assert(TPW <= 4, "wait_copies is written out for up to 4 tiles");
  static_assert(kTileBlocks * SROW <= TB, "the code tile is staged in the first x tile");
  __shared__ float red[WAVES];
  __shared__ float amax_sh;
  __shared__ __attribute__((aligned(1024))) char xlds_all[WAVES][TPW * TB];
  char* xlds = xlds_all[threadIdx.x >> 6];
  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * WAVES + wave_in_group();
  const int64_t nw = static_cast<int64_t>(gridDim.x) * WAVES;
  // counted into the barrier first: its add returns nothing and its load is
  // not waited for before the barrier
  unsigned long long leaf = 0;
  if (threadIdx.x < 64) leaf = arrive_wave0(ws);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    copy_tile_to_lds<B>(x, t < ntiles ? t : ntiles - 1, nblocks, xlds + i * TB);
  }
  // Tile i is rotated as soon as its own copies have landed, while the later
  // tiles' copies are still in flight.
  f32x4_t y[TPW][NM];
  float al[TPW];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    if (i == 0) wait_copies<(TPW - 1) * LdsTile<B>::kCopies>();
    if (i == 1) wait_copies<(TPW > 2 ? TPW - 2 : 0) * LdsTile<B>::kCopies>();
    if (i == 2) wait_copies<(TPW > 3 ? TPW - 3 : 0) * LdsTile<B>::kCopies>();
    if (i == 3) wait_copies<0>();
    uint4 xr[NK];
    read_tile_from_lds<B>(xlds + i * TB, xr);
    al[i] = ash_scale(column_sum_squares<B>(xr), sqrt_eb);
    float m = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const f32x4_t v = hadamard_mtile<B>(F, xr, mt);
      y[i][mt] = v;
      m = fmaxf(fmaxf(m, fabsf(v[0])), fabsf(v[1]));
      m = fmaxf(fmaxf(m, fabsf(v[2])), fabsf(v[3]));
    }
    if (t < ntiles && n < rv) amax = fmaxf(amax, m * (al[i] * Blk<B>::rsqrt_b));
  }
  // alpha after every tile's copies (a store in flight would count in the
  // waits above)
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    alpha[tc * kTileBlocks + (n < rv ? n : rv - 1)] = al[i];
  }
  const float wg = workgroup_max<WAVES>(amax, red);
  if (threadIdx.x < 64) {
    const float A = grid_max_wave0(wg, leaf, ws, spin_limit);
    if (threadIdx.x == 0) amax_sh = A;
  }
  __syncthreads();
  const float A = amax_sh;
  const float s = A == 0.0f ? 1.0f : kQmax / A;   // NaN stays NaN
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
  // x has been consumed: the first x tile of the wavefront stages its codes
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    if (t >= ntiles) continue;
    const float c = (al[i] * s) * Blk<B>::rsqrt_b;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(y[i][mt], c, mt, xlds);
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(xlds, q, t, rows_valid(t, nblocks));
    __builtin_amdgcn_wave_barrier();
  }
}

// The x-holding configurations stage x through LDS as well, in a ring of two
// tile slots per wavefront, since a workgroup's tiles (up to 256 KiB) do not
// fit in LDS at once: tile i + 2 is copied into tile i's slot as soon as tile
// i has moved into registers, so two tiles per wavefront are in flight until
// the last.  The tiles stay in registers as bf16 x across the barrier and are
// rotated again after it, as in compress_fused_kernel, whose arithmetic per
// tile (and so result) this is.  [8192, 3584] at B = 128, 4 tiles per
// wavefront, cold: 23.2 us with the direct loads (21.4 us of it remained
// with the barrier taken out, so the loads themselves were the cost), 19.8 us
// with the ring.
template <int B, int TPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void compress_fused_ring_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb, float* __restrict__ alpha,
    float* __restrict__ scale, char* __restrict__ ws, uint4* __restrict__ q, unsigned spin_limit) {
  constexpr int NK = B / 32, NM = B / 16, SROW = Blk<B>::kCodeRowMfma, TB = LdsTile<B>::kBytes;
  constexpr int S = 2, KC = LdsTile<B>::kCopies;
  static_assert(WAVES * S * TB <= 128 * 1024, "the ring exceeds the LDS budget");
  static_assert(TPW > S, "fewer tiles than slots: use compress_fused_lds_kernel");
  static_assert(kTileBlocks * SROW <= TB, "the code tile is staged in the first slot");
  __shared__ float red[WAVES];
  __shared__ float amax_sh;
  __shared__ __attribute__((aligned(1024))) char xlds_all[WAVES][S * TB];
  char* xlds = xlds_all[threadIdx.x >> 6];
  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * WAVES + wave_in_group();
  const int64_t nw = static_cast<int64_t>(gridDim.x) * WAVES;
  unsigned long long leaf = 0;
  if (threadIdx.x < 64) leaf = arrive_wave0(ws);
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int64_t t = wid + i * nw;
    copy_tile_to_lds<B>(x, t < ntiles ? t : ntiles - 1, nblocks, xlds + i * TB);
  }
  uint4 xr[TPW][NK];
  float al[TPW];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    // tiles issued after tile i: tile i + 1 (issued at tile i - 1), unless i is the last
    if (i + 1 < TPW) wait_copies<KC>(); else wait_copies<0>();
    read_tile_from_lds<B>(xlds + (i % S) * TB, xr[i]);
    if (i + S < TPW) {
      lds_reads_done();   // the slot is free once its reads have returned
      const int64_t tn = wid + (i + S) * nw;
      copy_tile_to_lds<B>(x, tn < ntiles ? tn : ntiles - 1, nblocks, xlds + (i % S) * TB);
    }
    al[i] = ash_scale(column_sum_squares<B>(xr[i]), sqrt_eb);
    float m = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      const f32x4_t v = hadamard_mtile<B>(F, xr[i], mt);
      m = fmaxf(fmaxf(m, fabsf(v[0])), fabsf(v[1]));
      m = fmaxf(fmaxf(m, fabsf(v[2])), fabsf(v[3]));
    }
    if (t < ntiles && n < rv) amax = fmaxf(amax, m * (al[i] * Blk<B>::rsqrt_b));
  }
  // alpha after every tile's copies (a store in flight would count in the
  // waits above)
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    alpha[tc * kTileBlocks + (n < rv ? n : rv - 1)] = al[i];
  }
  const float wg = workgroup_max<WAVES>(amax, red);
  if (threadIdx.x < 64) {
    const float A = grid_max_wave0(wg, leaf, ws, spin_limit);
    if (threadIdx.x == 0) amax_sh = A;
  }
  __syncthreads();
  const float A = amax_sh;
  const float s = A == 0.0f ? 1.0f : kQmax / A;   // NaN stays NaN
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    if (t >= ntiles) continue;
    const float c = (al[i] * s) * Blk<B>::rsqrt_b;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(hadamard_mtile<B>(F, xr[i], mt), c, mt, xlds);
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(xlds, q, t, rows_valid(t, nblocks));
    __builtin_amdgcn_wave_barrier();
  }
}

// ============================================================== decompress

// Rotation of one block in the wide layout (see the file header): index
// bits 0-2 lie in a chunk, bit 3 selects the chunk of a pair, bits 4-5 the
// quad lane and bits 6.. the 64-element group.  The butterflies visit the
// bits in the order 0-2, 5, 6.., 3, 4.  Any order gives the same transform in
// exact arithmetic; every kernel that rotates codes uses this one, so their
// fp32 results agree bitwise (decompress-sum and the fused
// decompress-sum-compress in particular).
template <int NA, bool FUSED = false>
__device__ __forceinline__ void rotate_wide(float (&v)[NA][8], const Quad& qd) {
#pragma unroll
  for (int a = 0; a < NA; ++a) fwht_chunk<1>(v[a]);
  fwht_quad_stage<NA, kQuadXor2, FUSED>(v, qd.c2);    // bit 5
  if constexpr (NA >= 4) fwht_chunk_stage<NA, 2>(v);  // bit 6
  if constexpr (NA >= 8) fwht_chunk_stage<NA, 4>(v);  // bit 7
  fwht_chunk_stage<NA, 1>(v);                         // bit 3
  fwht_quad_stage<NA, kQuadXor1, FUSED>(v, qd.c1);    // bit 4
}

// One block's codes in the wide layout (a block is 2 NA 16-byte pieces), one
// 16-byte load per 64-element group, kept as 8-code chunks (zero when !ok).
template <int NA>
__device__ __forceinline__ void load_codes_wide(const uint4* __restrict__ q, int64_t k, int ql, bool ok,
                                                uint2 (&c)[NA]) {
#pragma unroll
  for (int g = 0; g < NA / 2; ++g) {
    const uint4 v = ok ? load16<TACO_NT_Q_LOADS != 0>(&q[k * (2 * NA) + 4 * g + ql]) : make_uint4(0, 0, 0, 0);
    c[2 * g] = make_uint2(v.x, v.y);
    c[2 * g + 1] = make_uint2(v.z, v.w);
  }
}

// The bf16 values (times c) of a wide-layout tile into its LDS image: block
// blk of the tile in row blk (STRIDE bytes apart), its elements in order.
template <int NA, int STRIDE>
__device__ __forceinline__ void wide_tile_to_lds(const float (&v)[NA][8], float c, const Quad& qd, char* lds) {
#pragma unroll
  for (int a = 0; a < NA; ++a)
    *reinterpret_cast<uint4*>(lds + qd.blk * STRIDE + 128 * (a >> 1) + 32 * qd.ql + 16 * (a & 1)) =
        to_bf16x8(v[a], c);
}

template <int CTRL>
__device__ __forceinline__ uint4 dpp_u32x4(uint4 v) {
  return make_uint4(__builtin_amdgcn_mov_dpp(static_cast<int>(v.x), CTRL, 0xF, 0xF, true),
                    __builtin_amdgcn_mov_dpp(static_cast<int>(v.y), CTRL, 0xF, 0xF, true),
                    __builtin_amdgcn_mov_dpp(static_cast<int>(v.z), CTRL, 0xF, 0xF, true),
                    __builtin_amdgcn_mov_dpp(static_cast<int>(v.w), CTRL, 0xF, 0xF, true));
}

// Stores one block's bf16 values (times c) from the wide layout without LDS:
// the 16-byte pieces are exchanged across the quad first, so that each store
// instruction writes 64 contiguous bytes per quad (lane ql writes piece ql,
// then piece 4 + ql, of each 128-byte group; piece i belongs to lane i / 2).
template <int NA, bool NT>
__device__ __forceinline__ void store_wide_bf16(uint4* __restrict__ blk_out, const float (&v)[NA][8],
                                                float c, int ql, bool ok) {
  constexpr int kLow = 0x50, kHigh = 0xFA;   // DPP quad_perm [0,0,1,1] and [2,2,3,3]
  const bool odd = ql & 1;
#pragma unroll
  for (int g = 0; g < NA / 2; ++g) {
    const uint4 p0 = to_bf16x8(v[2 * g], c), p1 = to_bf16x8(v[2 * g + 1], c);
    const uint4 l0 = dpp_u32x4<kLow>(p0), l1 = dpp_u32x4<kLow>(p1);
    const uint4 h0 = dpp_u32x4<kHigh>(p0), h1 = dpp_u32x4<kHigh>(p1);
    if (ok) {
      store16<NT>(&blk_out[8 * g + ql], odd ? l1 : l0);
      store16<NT>(&blk_out[8 * g + 4 + ql], odd ? h1 : h0);
    }
  }
}

// LDS row stride of a tile's bf16 image on its way out (measured best of 0,
// 16, 32 and 64 bytes of padding).
template <int B>
constexpr int kOutStride = 2 * B + 32;

// Decompress: decode, rotate, multiply by 1/(alpha_k s sqrt(B)), round to
// bf16.  One tile per wavefront per trip, in the wide layout: one 16-byte
// code load per lane and 64-element group; the bf16 tile goes through the
// wavefront's LDS image and leaves lane-linearly, 1 KiB of whole cache lines
// per store instruction (direct stores of 64-byte half lines from the
// registers took 11.8 us instead of 8.9 on [4096, 4096], B = 128).  The grid
// holds at most kDecompressWgsPerCu<B> workgroups per CU and each wavefront
// walks its tiles (w, w + W, ...) as a software pipeline: the next tile's
// codes and scales are loaded before the current tile is rotated and stored.
// Loads and stores are branch-free (rows past the tensor's end load the last
// block and store duplicates of it), so that each wait is for the tile it
// needs.  Cold, against one batch of tiles per wavefront (U tiles' loads
// issued before any was used, U = 4 at B = 64, else 1): [4096, 1600] B = 64
// 6.2 -> 4.6 us, [4096, 4096] B = 128 9.1-9.2 -> 8.5-8.7 us, [8192, 3584]
// B = 128 15.3-16.0 -> 14.6 us, [4096, 4096] B = 256 9.9-10.1 -> 9.3-9.7 us.
// SBLK: `scale` holds one post-rotation scale per block (the per-block
// Dual-Scale variant) instead of one per tensor.
template <int B>
constexpr int kDecompressWgsPerCu = B == 64 ? 6 : 8;

// Lane-linear store of a tile's padded LDS image (ROW bytes per row, STRIDE
// apart) with every lane storing: rows past rows_valid store a copy of the
// last valid row to its own place (identical bytes), so no store is
// predicated.
template <int ROW, int STRIDE, bool NT>
__device__ __forceinline__ void lds_store_tile_clamped(const char* lds, uint4* __restrict__ g, int64_t tile,
                                                       int rows_valid) {
  constexpr int kChunksPerRow = ROW / 16, kChunks = kTileBlocks * kChunksPerRow;
  static_assert(kChunks % 64 == 0, "whole store instructions");
  const int lane = threadIdx.x & 63;
  uint4* base = g + tile * kChunks;
#pragma unroll
  for (int i = 0; i < kChunks / 64; ++i) {
    const int c = 64 * i + lane;
    const int r0 = c / kChunksPerRow, col = c % kChunksPerRow;
    const int r = r0 < rows_valid ? r0 : rows_valid - 1;
    store16<NT>(&base[r * kChunksPerRow + col], *reinterpret_cast<const uint4*>(lds + r * STRIDE + 16 * col));
  }
}

template <int B, bool SBLK>
__global__ __launch_bounds__(kThreads) void decompress_kernel(
    const uint4* __restrict__ q, const float* __restrict__ alpha, const float* __restrict__ scale,
    int64_t nblocks, uint4* __restrict__ out) {
  constexpr int NA = Blk<B>::NA, XS = kOutStride<B>;
  __shared__ __attribute__((aligned(16))) char lds_all[kWaves][kTileBlocks * XS];
  char* lds = lds_all[wave_in_group()];
  const Quad qd;
  const float s = SBLK ? 1.0f : *scale;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + wave_in_group();
  if (t >= ntiles) return;
  // Tile tt's codes, alpha and scale into (raw, al, sk); past the last tile
  // of this wavefront it loads tile `own` again (already in L2), not a new one.
  auto fetch = [&](int64_t tt, int64_t own, uint2 (&raw)[NA], float& al, float& sk)
      __attribute__((always_inline)) {
    const int64_t tc = tt < ntiles ? tt : own;
    const int rv = rows_valid(tc, nblocks);
    const int64_t k = tc * kTileBlocks + (qd.blk < rv ? qd.blk : rv - 1);
    load_codes_wide<NA>(q, k, qd.ql, true, raw);
    al = alpha[k];
    sk = SBLK ? scale[k] : s;
  };
  auto process = [&](int64_t tt, const uint2 (&raw)[NA], float al, float sk) __attribute__((always_inline)) {
    float v[NA][8];
#pragma unroll
    for (int a = 0; a < NA; ++a) from_fp8x8(raw[a], v[a]);
    // separate DPP moves: with the exchanges folded into the multiply-adds
    // (as in decompress-sum) [4096, 4096] at B = 128 measured 10.3 -> 10.4 us
    // cold, 10.45 -> 10.7 us with per-block scales
    rotate_wide<NA>(v, qd);
    wide_tile_to_lds<NA, XS>(v, (Blk<B>::rsqrt_b / (al * sk)) * qd.debt, qd, lds);
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_clamped<2 * B, XS, TACO_NT_OUT_STORES != 0>(lds, out, tt, rows_valid(tt, nblocks));
    __builtin_amdgcn_wave_barrier();
  };
  // two register sets, unrolled by two so that neither is copied
  uint2 ra[NA], rb[NA];
  float aa, ab, sa, sb;
  fetch(t, t, ra, aa, sa);
  while (true) {
    fetch(t + W, t, rb, ab, sb);
    __builtin_amdgcn_sched_barrier(0);   // the prefetch stays ahead of the rotation
    process(t, ra, aa, sa);
    t += W;
    if (t >= ntiles) break;
    fetch(t + W, t, ra, aa, sa);
    __builtin_amdgcn_sched_barrier(0);
    process(t, rb, ab, sb);
    t += W;
    if (t >= ntiles) break;
  }
}

struct Parts {
  const uint4* q[TACO_MAX_PARTS];
  const float* alpha[TACO_MAX_PARTS];
  const float* scale[TACO_MAX_PARTS];
};

// acc + d * w with the product rounded before the add (no fused
// multiply-add), so that a part and its exact negation cancel to zero, as the
// sum of their reconstructions does in exact arithmetic.
__device__ __forceinline__ float add_product(float acc, float d, float w) {
#pragma clang fp contract(off)
  return acc + d * w;
}

// The first part's product, as 0 + d * w would give it: one fused
// multiply-add with +0, so that an exact product -0 becomes +0 as it does
// when added to +0.  (The two differ only if a nonzero product rounded to
// -0, which needs w < 2^-141, far outside the input domain.)
__device__ __forceinline__ float first_product(float d, float w) { return fmaf(d, w, 0.0f); }

// An empty asm statement that takes the 8 values and gives them back: the
// compiler must have computed them where it stands (it emits no instruction).
__device__ __forceinline__ void pin_values(float (&v)[8]) {
  asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, expanded at compile
// time (a loop under #pragma unroll is left rolled past the unroller's size
// threshold, and its register arrays then go to scratch).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// acc += decode(codes) * w, chunk by chunk (FIRST: acc = decode(codes) * w,
// for the first part).
template <int NA, bool FIRST = false>
__device__ __forceinline__ void accumulate_chunks(float (&acc)[NA][8], const uint2 (&c)[NA], float w) {
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    float d[8];
    from_fp8x8(c[a], d);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[a][j] = FIRST ? first_product(d[j], w) : add_product(acc[a][j], d[j], w);
  }
}

// Decompress-and-sum.  The rotation is linear, so the parts are combined
// before it: acc = sum_p decode(q_p) / (alpha_{p,k} s_p), then one rotation
// and the 1/sqrt(B) factor.  This is the same sum as decompressing each part
// and adding the results, with P-1 fewer transforms per block.  Wide layout:
// each lane loads its 16 codes of every 64-element group with one 16-byte
// load per part, and the bf16 result leaves through store_wide_bf16 (staging
// it through LDS as decompress_kernel does measured slower with the earlier
// part loop, 21.5 -> 24.3 us for 4 parts, and with the one below the same at
// B = 128 and 256, 11.0 -> 10.55 us on [4096, 1600] at B = 64).  The parts
// are summed in order as their loads land, with DsumDepth<B, P> parts in
// flight ahead of the one being summed (the steps expanded at compile time
// and pinned, as in the decompress-sum-compress below): all of them at
// B = 64 and 128; one at B = 256, where a part takes 16 VGPRs per lane.  Before, every part was waited for before the first was
// summed (a branch around each load made the compiler wait for all of them).
// Cold, 4 parts: [4096, 1600] B = 64 11.4 -> 10.9 us, [4096, 4096] B = 128
// 22.4 -> 22.1 us, B = 256 22.3 -> 22.1 us; at B = 256 all parts in flight
// measured 23.6 us, and two or four tiles per wavefront (a grid of half or a
// quarter) 23.5 and 26.7 us.
template <int B, int P>
struct DsumDepth {
  static constexpr int value = B == 256 ? (P > 1 ? 1 : 0) : P - 1;
};

template <int B, int P>
__global__ __launch_bounds__(kThreads) void decompress_sum_kernel(
    Parts parts, int64_t nblocks, uint4* __restrict__ out) {
  constexpr int NA = Blk<B>::NA, C16 = Blk<B>::C16, D = DsumDepth<B, P>::value;
  const Quad qd;
  float part_scale[P];
#pragma unroll
  for (int p = 0; p < P; ++p)
    part_scale[p] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*parts.scale[p])));
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + wave_in_group(); t < ntiles; t += W) {
    const int64_t k = t * kTileBlocks + qd.blk;
    const bool ok = k < nblocks;
    // rows past the end load the last block (not stored): no branch around
    // a load, so that each part is waited for alone
    const int64_t kl = ok ? k : nblocks - 1;
    uint2 raw[D + 1][NA];
    float wt[D + 1];
    auto fetch = [&](const int p) __attribute__((always_inline)) {
      load_codes_wide<NA>(parts.q[p], kl, qd.ql, true, raw[p % (D + 1)]);
      wt[p % (D + 1)] = parts.alpha[p][kl];
    };
    static_for<D>([&](auto pc) __attribute__((always_inline)) { fetch(decltype(pc)::value); });
    float acc[NA][8];
    static_for<P>([&](auto pc) __attribute__((always_inline)) {
      constexpr int p = decltype(pc)::value;
      if constexpr (p + D < P) fetch(p + D);
      __builtin_amdgcn_sched_barrier(0);
      accumulate_chunks<NA, p == 0>(acc, raw[p % (D + 1)], 1.0f / (wt[p % (D + 1)] * part_scale[p]));
#pragma unroll
      for (int a = 0; a < NA; ++a) pin_values(acc[a]);
      __builtin_amdgcn_sched_barrier(0);
    });
    // The quad exchanges folded into the multiply-adds: cold, 4 parts of
    // [4096, 4096], B = 128 21.6 -> 21.3 us against exchanges through the LDS
    // crossbar (ds_swizzle), B = 256 21.75 -> 21.45 us per layer against
    // separate DPP moves (and 125 VGPRs instead of 144).
    rotate_wide<NA, true>(acc, qd);
    store_wide_bf16<NA, TACO_NT_SUM_STORES != 0>(out + k * C16, acc, Blk<B>::rsqrt_b * qd.debt, qd.ql, ok);
  }
}

// ============================================================== decompress-sum-compress
//
// The reduce-scatter local step with its result compressed again for the
// all-gather leg [TACO pt-summary, 2.B.3]: compress(decompress_sum(parts)).
// Fused when the reduced tensor's rotated blocks fit in the resident
// wavefronts' VGPRs: each wavefront sums its tiles' parts in the Hadamard
// domain and rounds to bf16 exactly as decompress_sum_kernel does (wide
// layout), re-lays the bf16 tile out through LDS into the MFMA operand
// layout, and continues as compress_fused_kernel (alpha, rotation on the
// matrix cores, grid-wide max, codes).  The bf16 sum never reaches HBM, and
// the result is bitwise equal to decompress_sum followed by compress.
//
// A tile's NP parts form a software pipeline: the tile's later parts' codes
// and alphas are loaded (up to dsc_depth of them ahead) while part p is
// decoded and weighed, and part p waits for its own loads only, so every
// wavefront keeps loads in flight while its vector ALUs work.  What keeps
// the compiler from undoing it:
// * the (tile, part) steps are expanded at compile time (static_for), so
//   every index is a constant;
// * the parts' scales are read once, up front (read at each part, through
//   pointers it cannot prove unwritten, they were vector loads, and their
//   wait covered the prefetched parts too);
// * each part's sums pass through pin_values, so that its adds are issued
//   before the next part's loads are waited for (left free, the compiler
//   deferred them into the next part and kept 32 products live: spills);
// * scheduling barriers on both sides of each part's accumulation.
// Cold, 4 parts, bitwise unchanged: [4096, 4096] B = 128 24.7-25.2 -> 23.5-
// 23.7 us with one part ahead, 22.9-23.2 us with three; [4096, 1600] B = 64
// 16.2 -> 14.0 us; [256, 1024] B = 64 8.1 -> 7.6 us.  The next tile's first
// parts load while this tile is rotated: 23.8-24.3 -> 23.3-23.5 us on
// [4096, 4096] (same device, back to back), 14.0 -> 13.9 us on [4096, 1600].

// Parts in flight ahead of the one being summed in decompress_sum_compress_
// kernel: the rest of the tile's, up to three, and fewer where that would
// spill (B = 128 with two tiles per wavefront, which holds y for the first
// tile while it sums the second).
template <int B, int TPW, int NP>
constexpr int dsc_depth() {
  if (B == 128 && TPW == 2 && NP > 4) return NP > 6 ? 1 : 2;
  return NP - 1 < 3 ? NP - 1 : 3;
}

template <int B, int TPW, int WAVES, int NP>
__global__ __launch_bounds__(64 * WAVES) void decompress_sum_compress_kernel(
    Parts parts, int64_t nblocks, float sqrt_eb, float* __restrict__ alpha,
    float* __restrict__ scale, char* __restrict__ ws, uint4* __restrict__ q, unsigned spin_limit) {
  static_assert(NP >= 1 && NP <= TACO_MAX_PARTS, "part count");
  constexpr int NA = Blk<B>::NA, NK = B / 32, NM = B / 16;
  constexpr int XROW = 2 * B + 16, SROW = Blk<B>::kCodeRowMfma;
  constexpr int kLdsWave = kTileBlocks * (XROW > SROW ? XROW : SROW);
  __shared__ float red[WAVES];
  __shared__ float amax_sh;
  __shared__ __attribute__((aligned(16))) char lds_all[WAVES][kLdsWave];
  char* lds = lds_all[wave_in_group()];   // a scalar register, not a VGPR held to the stores
  const Quad qd;
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * WAVES + wave_in_group();
  const int64_t nw = static_cast<int64_t>(gridDim.x) * WAVES;
  // Counted into the barrier first (the adds return nothing); the count is
  // loaded with the last tile, while its rotations run, so that it occupies
  // no register during the accumulation.
  if (threadIdx.x < 64) arrive_add_wave0(ws);
  unsigned long long leaf = 0;
  float part_scale[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p)
    part_scale[p] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*parts.scale[p])));
  f32x4_t y[TPW][NM];
  float al_r[TPW];
  float amax = 0.0f;
  auto finish_tile = [&](const int i, float (&acc)[NA][8]) __attribute__((always_inline)) {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    if (i == TPW - 1) leaf = leaf_count(ws);
    // quad exchanges folded into the multiply-adds: 21.8 -> 21.3 us cold
    // (4 parts, [4096, 4096], B = 128) against exchanges through the LDS
    // crossbar, which had been 1.1 us faster than separate DPP moves
    rotate_wide<NA, true>(acc, qd);
    const float r = Blk<B>::rsqrt_b * qd.debt;
    wide_tile_to_lds<NA, XROW>(acc, r, qd, lds);
    __builtin_amdgcn_wave_barrier();
    // The MFMA operand is read from LDS one K-step at a time (few live
    // registers); every sum is accumulated in the same order as
    // column_sum_squares and hadamard_mtile, so the values are identical.
    const HadFrag F = make_hadamard_fragments();
    constexpr int kChains = NK >= 4 ? 4 : 2;
    float ssq[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) ssq[c] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) y[i][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const uint4 xk = *reinterpret_cast<const uint4*>(lds + n * XROW + 64 * kt + 16 * g);
      float& sc = ssq[kt % kChains];
      sc = dot2_bf16(xk.x, xk.x, sc);
      sc = dot2_bf16(xk.y, xk.y, sc);
      sc = dot2_bf16(xk.z, xk.z, sc);
      sc = dot2_bf16(xk.w, xk.w, sc);
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const bool neg = __builtin_popcount((mt >> 1) & kt) & 1;
        const bf16x8_t a = neg ? F.neg[mt & 1] : F.pos[mt & 1];
        y[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, xk), y[i][mt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_wave_barrier();
    float ss = ssq[0];
#pragma unroll
    for (int c = 1; c < kChains; ++c) ss += ssq[c];
    const float al = ash_scale(column_sum_rows(ss), sqrt_eb);
    al_r[i] = al;
    alpha[tc * kTileBlocks + (n < rv ? n : rv - 1)] = al;
    float m = 0.0f;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) {
      m = fmaxf(fmaxf(m, fabsf(y[i][mt][0])), fabsf(y[i][mt][1]));
      m = fmaxf(fmaxf(m, fabsf(y[i][mt][2])), fabsf(y[i][mt][3]));
    }
    if (t < ntiles && n < rv) amax = fmaxf(amax, m * (al * Blk<B>::rsqrt_b));
  };
  auto block_of = [&](const int i) __attribute__((always_inline)) -> int64_t {
    const int64_t t = wid + i * nw;
    const int64_t tc = t < ntiles ? t : ntiles - 1;
    const int rv = rows_valid(tc, nblocks);
    return tc * kTileBlocks + (qd.blk < rv ? qd.blk : rv - 1);
  };
  constexpr int NI = TPW * NP, D = dsc_depth<B, TPW, NP>(), NB = D + 1;
  uint2 raw[NB][NA];
  float ra[NB];
  auto fetch = [&](const int it) __attribute__((always_inline)) {
    const int i = it / NP, p = it % NP;
    const int64_t kq = block_of(i);
    load_codes_wide<NA>(parts.q[p], kq, qd.ql, true, raw[it % NB]);
    ra[it % NB] = parts.alpha[p][kq];
  };
  // a tile's first D parts (the next tile's before this one is rotated), then
  // part p + D while part p is summed
  static_for<D>([&](auto c) __attribute__((always_inline)) { fetch(decltype(c)::value); });
  float acc[NA][8];
  static_for<NI>([&](auto item) __attribute__((always_inline)) {
    constexpr int it = decltype(item)::value, i = it / NP, p = it % NP;
    if constexpr (p + D < NP) fetch(it + D);
    __builtin_amdgcn_sched_barrier(0);
    const float w = 1.0f / (ra[it % NB] * part_scale[p]);
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      float d[8];
      from_fp8x8(raw[it % NB][a], d);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[a][e] = p == 0 ? first_product(d[e], w) : add_product(acc[a][e], d[e], w);
    }
#pragma unroll
    for (int a = 0; a < NA; ++a) pin_values(acc[a]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (p == NP - 1) {
      // the next tile's first D parts load while this tile is rotated
      static_for<D>([&](auto c) __attribute__((always_inline)) {
        if constexpr (it + 1 + decltype(c)::value < NI) fetch(it + 1 + decltype(c)::value);
      });
      __builtin_amdgcn_sched_barrier(0);
      finish_tile(i, acc);
    }
  });
  const float wg = workgroup_max<WAVES>(amax, red);
  if (threadIdx.x < 64) {
    const float A = grid_max_wave0(wg, leaf, ws, spin_limit);
    if (threadIdx.x == 0) amax_sh = A;
  }
  __syncthreads();
  const float A = amax_sh;
  const float s = A == 0.0f ? 1.0f : kQmax / A;   // NaN stays NaN
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int64_t t = wid + i * nw;
    if (t >= ntiles) continue;
    const float c = (al_r[i] * s) * Blk<B>::rsqrt_b;
#pragma unroll
    for (int mt = 0; mt < NM; ++mt) codes_to_lds_mfma<B>(y[i][mt], c, mt, lds);
    __builtin_amdgcn_wave_barrier();
    lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(lds, q, t, rows_valid(t, nblocks));
    __builtin_amdgcn_wave_barrier();
  }
}

// ============================================================== single-pass Dual-Scale variants
//
// Dual-Scale variants whose scales need no tensor-wide maximum, so that
// compression is one streaming kernel without a grid-wide barrier, the single
// fused kernel the pages describe [TACO pt-summary, 2.B.2 and 2.B.3]:
//   kDsBlockGuard  a per-block post-rotation scale, s_k = 448 / max|y_k| when
//                  the block would overflow and 1 otherwise, stored per block;
//   kDsDelayed     the per-tensor s = 448 / amax_prev of an earlier tensor,
//                  rotated values beyond the range saturating at +-448; this
//                  tensor's maximum is folded into kAmaxSlots words of amax_out
//                  (atomic max at slot workgroup mod kAmaxSlots; the slots lie
//                  on separate 256-byte lines, since atomics to one line
//                  serialise: 16.6 us with contiguous slots, 12.4 us spread,
//                  with the atomic issued before the code stores and 8
//                  wavefronts per workgroup) for the next call.
// One tile per wavefront; the arithmetic per tile is the per-tensor path's
// (MFMA rotation of raw x, alpha from the same registers).
constexpr int kDsBlockGuard = 1;
constexpr int kDsDelayed = 2;
constexpr int kAmaxSlots = TACO_AMAX_SLOTS;
constexpr int kAmaxStride = TACO_AMAX_FLOATS / TACO_AMAX_SLOTS;   // one slot per 256-byte line

// Max over the 4 lanes of an MFMA column (lanes n, n+16, n+32, n+48): every
// lane of the column gets it.
__device__ __forceinline__ float column_max(float v) {
  const unsigned u = __float_as_uint(v);
  const auto p32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
  const unsigned w = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
}

template <int B, int MODE, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void compress_streaming_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float sqrt_eb, const float* __restrict__ amax_prev,
    float* __restrict__ alpha, float* __restrict__ scale, unsigned* __restrict__ amax_out,
    uint4* __restrict__ q) {
  constexpr int NK = B / 32, NM = B / 16, SROW = Blk<B>::kCodeRowMfma;
  __shared__ float red[WAVES];
  constexpr int TB = LdsTile<B>::kBytes;
  static_assert(kTileBlocks * SROW <= TB, "codes staged in the x tile");
  __shared__ __attribute__((aligned(1024))) char lds_all[WAVES][TB];
  char* lds = lds_all[threadIdx.x >> 6];
  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, n = lane & 15;
  const int64_t ntiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * WAVES + wave_in_group();
  const int64_t tc = t < ntiles ? t : ntiles - 1;
  const int rv = rows_valid(tc, nblocks);
  const int row = n < rv ? n : rv - 1;
  uint4 xr[NK];
  // x through LDS (1 KiB of whole cache lines per copy instruction, as in
  // the fused kernels), then into the MFMA operand registers; the tile's
  // region stages the codes afterwards.  [4096, 4096] at B = 128, cold:
  // per-block guard 11.8 -> 10.7 us, delayed scale 13.7 -> 11.9 us
  // ([8192, 3584]: 19.2 -> 16.8 and 21.1 -> 20.2 us) against loading x
  // straight into the operand layout.
  copy_tile_to_lds<B>(x, tc, nblocks, lds);
  wait_copies<0>();
  read_tile_from_lds<B>(lds, xr);
  float s = 1.0f;
  if constexpr (MODE == kDsDelayed) {
    static_assert(kAmaxSlots == 64, "one amax slot per lane");
    const float prev = wave_max(amax_prev[lane * kAmaxStride]);
    s = prev > 0.0f ? kQmax / prev : 1.0f;
  }
  const float al = ash_scale(column_sum_squares<B>(xr), sqrt_eb);
  alpha[tc * kTileBlocks + row] = al;              // duplicates write identical values
  f32x4_t y[NM];
  float m = 0.0f;
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    y[mt] = hadamard_mtile<B>(F, xr, mt);
    m = fmaxf(fmaxf(m, fabsf(y[mt][0])), fabsf(y[mt][1]));
    m = fmaxf(fmaxf(m, fabsf(y[mt][2])), fabsf(y[mt][3]));
  }
  const float bmax = column_max(m) * (al * Blk<B>::rsqrt_b);     // max |y| of the block
  if constexpr (MODE == kDsBlockGuard) {
    s = bmax > kQmax ? kQmax / bmax : 1.0f;
    scale[tc * kTileBlocks + row] = s;
  }
  if constexpr (MODE == kDsDelayed) {
    // issued before the code stores, so that its latency overlaps them
    const float wg = workgroup_max<WAVES>(t < ntiles && n < rv ? bmax : 0.0f, red);
    if (threadIdx.x == 0)
      __hip_atomic_fetch_max(&amax_out[(blockIdx.x % kAmaxSlots) * kAmaxStride], __float_as_uint(wg),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const float c = (al * s) * Blk<B>::rsqrt_b;
  const int g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < NM; ++mt) {
    // saturate before the conversion
    const float v0 = fminf(fmaxf(y[mt][0] * c, -kQmax), kQmax), v1 = fminf(fmaxf(y[mt][1] * c, -kQmax), kQmax);
    const float v2 = fminf(fmaxf(y[mt][2] * c, -kQmax), kQmax), v3 = fminf(fmaxf(y[mt][3] * c, -kQmax), kQmax);
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, wd, true);
    *reinterpret_cast<int*>(lds + n * SROW + 16 * mt + 4 * g) = wd;
  }
  __builtin_amdgcn_wave_barrier();
  if (t < ntiles) lds_store_tile_to_global<B, SROW, TACO_NT_CODE_STORES != 0>(lds, q, t, rv);
  __builtin_amdgcn_wave_barrier();
  if constexpr (MODE == kDsDelayed)
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
}

// ============================================================== INT8 degrade path
//
// Symmetric absmax INT8: the comparator the pages argue against [TACO
// pt-summary, sections 1 and 2.A: uniform INT8 steps send the dense
// near-zero values of TP tensors to the same integer] and a fallback for
// consumers without FP8.  A = max|x| over the tensor or over a block of B
// consecutive elements of a row, s = fp32(127 / A) (1 if A = 0),
// code = clamp(round_half_even(x s)), +-127) of the exact product, and
// x_hat = bf16_RNE(code / s) of the exact quotient: both roundings are
// decided exactly (int8_code, int8_to_bf16), not on an fp32 intermediate.
// No ASH and no rotation.  Streaming kernels: each lane owns 8 consecutive
// bf16 values (one 16-byte load) and their 8 codes (one 8-byte store); a
// workgroup covers kInt8Unroll x 256 consecutive 16-byte pieces per trip.

constexpr int kInt8Unroll = 4;

// Keeps a trip's loads ahead of every use of them: without it the scheduler
// may place the first use right after the first load, and the wait for it
// then holds back the issue of the others.
__device__ __forceinline__ void all_loads_issued() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// max |x| of 8 bf16 values as a bf16 bit pattern (non-negative bf16 values
// order like their bits).
__device__ __forceinline__ unsigned bf16x8_absmax_bits(const uint4 v) {
  const unsigned a = max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu);
  const unsigned b = max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu);
  const unsigned c = max(v.z & 0x7FFFu, (v.z >> 16) & 0x7FFFu);
  const unsigned d = max(v.w & 0x7FFFu, (v.w >> 16) & 0x7FFFu);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float int8_scale_of(float amax) {
  return amax == 0.0f ? 1.0f : 127.0f / amax;
}

// clamp(round_half_even(x s), +-127) of the exact product.  p = fp32(x s) and
// e = x s - p exactly (one fma: x has at most 8 significant bits and s 24, so
// the product has at most 32 and the residual fits in fp32).  rint(p) can
// differ from the exact rounding only where p lies exactly half-way between
// two integers while x s does not (rounding to fp32 moves a value onto a
// half-integer, never across one); there the sign of e decides.  Contraction
// is off: fusing x * s into p - r would change the half-way test.
__device__ __forceinline__ float int8_code(float x, float s) {
#pragma clang fp contract(off)
  const float p = x * s;
  const float e = fmaf(x, s, -p);
  const float r = __builtin_rintf(p);
  const float d = p - r;
  const float adj = (d == 0.5f && e > 0.0f) ? 1.0f : ((d == -0.5f && e < 0.0f) ? -1.0f : 0.0f);
  return fminf(fmaxf(r + adj, -127.0f), 127.0f);
}

// The same code when the fp32 product is not exactly half-way between two
// integers: then rint(fp32(x s)) is the exact rounding.
__device__ __forceinline__ float int8_code_fast(float x, float s) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(x * s), -127.0f, 127.0f);
}

// Whether any of the 8 bf16 values in v has an fp32 product with s that lies
// exactly half-way between two integers (the only case int8_code_fast can get
// wrong).
__device__ __forceinline__ bool int8_half_way(const uint4 v, float s) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  bool h = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h |= __builtin_amdgcn_fractf(__uint_as_float(w[i] << 16) * s) == 0.5f;
    h |= __builtin_amdgcn_fractf(__uint_as_float(w[i] & 0xFFFF0000u) * s) == 0.5f;
  }
  return h;
}

// The two int8 codes of the bf16 pair in w, in the low 16 bits (element 0 first).
template <bool EXACT>
__device__ __forceinline__ unsigned int8_pair(unsigned w, float s) {
  const float a = __uint_as_float(w << 16), b = __uint_as_float(w & 0xFFFF0000u);
  const float lo = EXACT ? int8_code(a, s) : int8_code_fast(a, s);
  const float hi = EXACT ? int8_code(b, s) : int8_code_fast(b, s);
  return (static_cast<unsigned>(static_cast<int>(lo)) & 0xFFu) |
         ((static_cast<unsigned>(static_cast<int>(hi)) & 0xFFu) << 8);
}

template <bool EXACT>
__device__ __forceinline__ uint2 int8_codes_bf16x8(const uint4 v, float s) {
  return make_uint2(int8_pair<EXACT>(v.x, s) | (int8_pair<EXACT>(v.y, s) << 16),
                    int8_pair<EXACT>(v.z, s) | (int8_pair<EXACT>(v.w, s) << 16));
}

// The 8 codes of a 16-byte piece: fp32 products decide them unless one of the
// wavefront's products lies exactly half-way between two integers (rare),
// and then the wavefront decides this piece on the exact products.
__device__ __forceinline__ uint2 int8_codes_piece(const uint4 v, float s) {
  if (__builtin_amdgcn_ballot_w64(int8_half_way(v, s)) != 0) return int8_codes_bf16x8<true>(v, s);
  return int8_codes_bf16x8<false>(v, s);
}

// bf16_RNE(c / s) of the exact quotient, for an integer code c and s > 0
// (r = fp32(1 / s)).  |c| r lies within 2^-23 (relative) of |c| / s, far
// inside half a bf16 step, so the correctly rounded bf16 value is the
// truncation t of |c| r or its successor.  The midpoint m between them is an
// fp32 value, and |c| - m s, formed by one fma (exact product, one rounding),
// has the sign of |c| / s - m: above m rounds up, exactly m rounds to the
// even one of the two.
__device__ __forceinline__ unsigned int8_to_bf16(int c, float s, float r) {
  const float a = static_cast<float>(c < 0 ? -c : c);
  const unsigned t = __float_as_uint(a * r) >> 16;
  const float m = __uint_as_float((t << 16) | 0x8000u);
  const float d = fmaf(-m, s, a);
  const unsigned up = (d > 0.0f || (d == 0.0f && (t & 1u))) ? 1u : 0u;
  return (t + up) | (c < 0 ? 0x8000u : 0u);
}

// The 8 codes of c as fp32 values.
__device__ __forceinline__ void int8x8_values(const uint2 c, float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = static_cast<float>(static_cast<int8_t>((c.x >> (8 * j)) & 0xFFu));
    v[4 + j] = static_cast<float>(static_cast<int8_t>((c.y >> (8 * j)) & 0xFFu));
  }
}

// Whether any fp32 product code * r of the 8 codes lies within 3 fp32 steps
// of a bf16 midpoint (low 16 bits within 0x8000 +- 3).  |code| r is within 2
// steps of |code| / s, so elsewhere the bf16 rounding of the fp32 product is
// the rounding of the exact quotient.
__device__ __forceinline__ bool int8_near_midpoint(const float (&v)[8], float r) {
  bool near = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) near |= ((__float_as_uint(v[j] * r) & 0xFFFFu) - 0x7FFDu) < 7u;
  return near;
}

template <bool EXACT>
__device__ __forceinline__ uint4 bf16x8_from_int8x8(const float (&v)[8], float s, float r) {
  if constexpr (!EXACT) return to_bf16x8(v, r);
  unsigned h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = int8_to_bf16(static_cast<int>(v[j]), s, r);
  return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// The 8 bf16 outputs of a piece of codes: the bf16 rounding of the fp32
// product code * r is the correctly rounded quotient unless a product of the
// wavefront lies near a bf16 midpoint (rare), and then the wavefront decides
// this piece exactly.
__device__ __forceinline__ uint4 bf16_piece_from_int8(const uint2 c, float s, float r) {
  float v[8];
  int8x8_values(c, v);
  if (__builtin_amdgcn_ballot_w64(int8_near_midpoint(v, r)) != 0) return bf16x8_from_int8x8<true>(v, s, r);
  return bf16x8_from_int8x8<false>(v, s, r);
}

// Per-tensor INT8, pass 1: each workgroup's max |x| into partial[blockIdx.x].
__global__ __launch_bounds__(kThreads) void int8_absmax_kernel(const uint4* __restrict__ x, int64_t n16,
                                                               float* __restrict__ partial) {
  __shared__ float red[kWaves];
  unsigned m = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kInt8Unroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kInt8Unroll; base < n16; base += stride) {
    uint4 v[kInt8Unroll];
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      v[u] = x[i < n16 ? i : n16 - 1];      // branch-free: past the end, a copy of the last piece
    }
    all_loads_issued();
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) m = max(m, bf16x8_absmax_bits(v[u]));
  }
  const float wg = workgroup_max<kWaves>(__uint_as_float(m << 16), red);
  if (threadIdx.x == 0) partial[blockIdx.x] = wg;
}

// Per-tensor INT8, pass 2: every workgroup folds the partial maxima into s,
// then converts its pieces.
__global__ __launch_bounds__(kThreads) void int8_quant_tensor_kernel(
    const uint4* __restrict__ x, int64_t n16, const float* __restrict__ partial, int npartial,
    float* __restrict__ scale, uint2* __restrict__ q) {
  __shared__ float red[kWaves];
  float m = 0.0f;
  for (int p = threadIdx.x; p < npartial; p += kThreads) m = fmaxf(m, partial[p]);
  const float s = int8_scale_of(workgroup_max<kWaves>(m, red));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kInt8Unroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kInt8Unroll; base < n16; base += stride) {
    uint4 v[kInt8Unroll];
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      v[u] = x[i < n16 ? i : n16 - 1];      // branch-free: past the end, a copy of the last piece
    }
    all_loads_issued();
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      const uint2 c = int8_codes_piece(v[u], s);
      store8<TACO_NT_CODE_STORES != 0>(&q[i < n16 ? i : n16 - 1], c);   // past the end: the last piece again
    }
  }
}

// Per-block INT8: a block spans G = B / 8 consecutive lanes (G divides 64 and
// every trip starts on a wavefront boundary, so no block straddles two
// wavefronts); its max is an xor-shuffle over the group.  The trip loop is
// uniform over the workgroup, and a group lies entirely inside or outside
// the tensor, so the shuffles of a group inside it only read lanes of the
// same group.  A group outside it loads the tensor's last block (lane j of
// the group its piece j), so it derives that block's scale and codes and
// stores them again, unchanged, in place: no branch surrounds a store, which
// would make the compiler wait for every load in flight at its join (cold,
// [4096, 4096] at B = 128: 12.80 -> 11.70 us; the same change took the
// per-tensor codes 16.1 -> 15.8 us and the decompressions 9.14 -> 8.55 and
// 8.87 -> 8.42 us).
template <int G>
__global__ __launch_bounds__(kThreads) void int8_quant_block_kernel(
    const uint4* __restrict__ x, int64_t n16, float* __restrict__ scale, uint2* __restrict__ q) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kInt8Unroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kInt8Unroll; base < n16; base += stride) {
    uint4 v[kInt8Unroll];
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      v[u] = x[i < n16 ? i : n16 - G + lane % G];      // past the end: the last block again
    }
    all_loads_issued();
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      const int64_t ic = i < n16 ? i : n16 - G + lane % G;
      unsigned m = bf16x8_absmax_bits(v[u]);
#pragma unroll
      for (int o = 1; o < G; o <<= 1) m = max(m, static_cast<unsigned>(__shfl_xor(static_cast<int>(m), o)));
      const float s = int8_scale_of(__uint_as_float(m << 16));
      const uint2 c = int8_codes_piece(v[u], s);
      store8<TACO_NT_CODE_STORES != 0>(&q[ic], c);
      scale[ic / G] = s;                    // the group's lanes store the same value
    }
  }
}

// INT8 decompress.  G = B / 8 lanes per scale block, or 0 for one scale per
// tensor.
template <int G>
__global__ __launch_bounds__(kThreads) void int8_dequant_kernel(
    const uint2* __restrict__ q, const float* __restrict__ scale, int64_t n16, uint4* __restrict__ out) {
  const float s0 = G == 0 ? *scale : 1.0f;
  const float r0 = 1.0f / s0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kInt8Unroll;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kInt8Unroll; base < n16; base += stride) {
    uint2 c[kInt8Unroll];
    float sk[kInt8Unroll];
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      const int64_t ic = i < n16 ? i : n16 - 1;   // branch-free loads, as above
      c[u] = q[ic];
      if constexpr (G != 0) sk[u] = scale[ic / G];
      else sk[u] = 1.0f;
    }
    all_loads_issued();
#pragma unroll
    for (int u = 0; u < kInt8Unroll; ++u) {
      const int64_t i = base + u * kThreads + threadIdx.x;
      const uint4 o = G == 0 ? bf16_piece_from_int8(c[u], s0, r0) : bf16_piece_from_int8(c[u], sk[u], 1.0f / sk[u]);
      store16<TACO_NT_OUT_STORES != 0>(&out[i < n16 ? i : n16 - 1], o);   // past the end: the last piece again
    }
  }
}

// ----------------------------------------------------------------- host side

constexpr int kMaxDevices = 64;

// A launch limit of the current device, computed once per device: CU counts
// and residency differ between GPU models, so a value cached for the whole
// process would be wrong for a second, different GPU.  cache[dev] is 0 until
// computed; compute() returns a positive value, or a value <= 0 (not cached)
// when the query fails.  Threads that race on a first call compute the same
// value.
template <typename F>
int per_device(std::atomic<int> (&cache)[kMaxDevices], F compute) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return compute();
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    v = compute();
    if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

int device_cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  return per_device(cache, [] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    return n;
  });
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool block_ok(int32_t b) { return b == 64 || b == 128 || b == 256; }

taco_status_t check_shape(int64_t tokens, int64_t hidden, int32_t block) {
  if (tokens < 1 || hidden < 1) return TACO_ERR_SHAPE;
  if (!block_ok(block)) return TACO_ERR_UNSUPPORTED_BLOCK;
  if (hidden % block != 0) return TACO_ERR_SHAPE;
  // keep the element count well inside 64-bit index arithmetic
  if (tokens > (int64_t(1) << 40) / hidden) return TACO_ERR_SHAPE;
  return TACO_OK;
}

// Workgroups of one-tile-per-wavefront kernels (the grid-stride loops cover
// any tiles beyond).
int tile_grid(int64_t nblocks) {
  const int64_t tiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t g = (tiles + kWaves - 1) / kWaves;
  return static_cast<int>(std::min<int64_t>(std::max<int64_t>(g, 1), INT32_MAX));
}

// Workgroups of `kernel` that fit on the whole device at once.
template <typename Kernel>
int resident_grid(Kernel kernel, int threads) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int cus = device_cu_count();
  return per_cu * (cus > 0 ? cus : 256);
}

taco_status_t launched() { return hipGetLastError() == hipSuccess ? TACO_OK : TACO_ERR_HIP; }


// Launches the fused compress with TPW tiles per wavefront if every one of its
// wavefronts can be resident at once (and the barrier has leaves for them).
// (With launch false it only reports whether the configuration fits.)
// At most one workgroup per CU: at B = 64 with one tile per wavefront two
// 16-wavefront workgroups fit on a CU, but that grid measured slower than
// two tiles per wavefront on one workgroup per CU ([4096, 1600]: 400
// workgroups 9.9 us, 200 workgroups 9.1-9.3 us, 256 workgroups with the
// tiles spread unevenly 9.4 us, cold).
int fused_grid_cap(int resident) {
  const int cus = device_cu_count();
  return std::min({resident, cus > 0 ? cus : resident, kMaxSlots});
}

template <int B, int TPW, bool HOLD_Y, int WAVES>
bool try_fused(const uint4* x, int64_t nblocks, float sqrt_eb, float* alpha, float* scale, char* ws,
               uint4* q, hipStream_t stream, bool launch, unsigned polls) {
  const int64_t tiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t g = ((tiles + TPW - 1) / TPW + WAVES - 1) / WAVES;
  if constexpr (HOLD_Y && TACO_FUSED_LDS != 0) {   // y held: x staged through LDS
    static std::atomic<int> caps[kMaxDevices];
    const int cap = per_device(caps, [] { return fused_grid_cap(resident_grid(compress_fused_lds_kernel<B, TPW, WAVES>, 64 * WAVES)); });
    if (g > cap) return false;
    if (launch)
      hipLaunchKernelGGL((compress_fused_lds_kernel<B, TPW, WAVES>), dim3(g), dim3(64 * WAVES), 0,
                         stream, x, nblocks, sqrt_eb, alpha, scale, ws, q, polls);
  } else if constexpr (!HOLD_Y && TACO_FUSED_LDS != 0) {   // x held, staged through an LDS ring
    static std::atomic<int> caps[kMaxDevices];
    const int cap = per_device(caps, [] { return fused_grid_cap(resident_grid(compress_fused_ring_kernel<B, TPW, WAVES>, 64 * WAVES)); });
    if (g > cap) return false;
    if (launch)
      hipLaunchKernelGGL((compress_fused_ring_kernel<B, TPW, WAVES>), dim3(g), dim3(64 * WAVES), 0,
                         stream, x, nblocks, sqrt_eb, alpha, scale, ws, q, polls);
  } else {
    static std::atomic<int> caps[kMaxDevices];
    const int cap = per_device(caps, [] { return fused_grid_cap(resident_grid(compress_fused_kernel<B, TPW, HOLD_Y, WAVES>, 64 * WAVES)); });
    if (g > cap) return false;
    if (launch)
      hipLaunchKernelGGL((compress_fused_kernel<B, TPW, HOLD_Y, WAVES>), dim3(g), dim3(64 * WAVES), 0,
                         stream, x, nblocks, sqrt_eb, alpha, scale, ws, q, polls);
  }
  return true;
}

// Fused configurations, fewest tiles per wavefront first.  Holding the
// rotated blocks (fp32 y, at most 64 of the 128 VGPRs a lane has at 16
// wavefronts per CU) covers 64 MiB of y, e.g. [4096, 4096] at B = 128.
// Beyond that the wavefronts hold the bf16 input instead (half the registers
// per element) and rotate it again after the barrier, which covers 1.5 to 2
// times as much: [8192, 4096] at B = 128 or 256, [8192, 3072] at B = 64.
// Larger tensors take the two-pass path.  Every variant issues the same
// MFMA sequence per tile, so all give identical results.  With one tile per
// wavefront, workgroups of 4 or 8 wavefronts come first, so that a small
// tensor spreads over up to four times as many CUs (each workgroup still on
// a CU of its own): cold, [256, 1024] at B = 64 5.24 -> 4.90 us,
// [1024, 4096] at B = 128 7.86 -> 7.60 us.
template <int B>
bool launch_fused(const uint4* x, int64_t nblocks, float sqrt_eb, float* alpha, float* scale, char* ws,
                  uint4* q, hipStream_t stream, bool launch, unsigned polls) {
  if (try_fused<B, 1, true, kWavesC / 4>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  if (try_fused<B, 1, true, kWavesC / 2>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  if (try_fused<B, 1, true, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  if constexpr (B <= 128)
    if (try_fused<B, 2, true, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  if constexpr (B == 64) {
    if (try_fused<B, 4, true, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
    if (try_fused<B, 6, false, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  }
  if constexpr (B == 128) {
    if (try_fused<B, 3, false, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
    if (try_fused<B, 4, false, kWavesC>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  }
  if constexpr (B == 256)   // 8 wavefronts per CU: 226 VGPRs
    if (try_fused<B, 4, false, kWavesC / 2>(x, nblocks, sqrt_eb, alpha, scale, ws, q, stream, launch, polls)) return true;
  return false;
}

template <int B>
void launch_compress(const void* x, int64_t nblocks, float energy, uint8_t* q, float* alpha,
                     float* scale, void* workspace, hipStream_t stream, bool single_pass, unsigned polls) {
  const float sqrt_eb = static_cast<float>(sqrt(static_cast<double>(energy) * B));
  const uint4* xv = static_cast<const uint4*>(x);
  uint4* qv = reinterpret_cast<uint4*>(q);
  char* ws = static_cast<char*>(workspace);
  float* partial = reinterpret_cast<float*>(ws + kPartialOffset);
  // Single fused pass when the tensor fits in the resident wavefronts' VGPRs.
  if (single_pass && launch_fused<B>(xv, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, true, polls)) return;
  constexpr int U = 2;
  const int64_t tiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t per_wg = static_cast<int64_t>(kWaves) * U;
  const int64_t want = (tiles + per_wg - 1) / per_wg;
  const int gs = static_cast<int>(std::min<int64_t>(want, kMaxPartials));
  const int gq = static_cast<int>(std::min<int64_t>(want, INT32_MAX));
  hipLaunchKernelGGL((compress_stats_mfma_kernel<B, U>), dim3(gs), dim3(kThreads), 0, stream,
                     xv, nblocks, sqrt_eb, alpha, partial);
  hipLaunchKernelGGL((compress_quant_mfma_kernel<B, U>), dim3(gq), dim3(kThreads), 0, stream,
                     xv, nblocks, sqrt_eb, partial, gs, scale, qv);
}

template <int B, bool SBLK>
void launch_decompress(const uint8_t* q, const float* alpha, const float* scale, int64_t nblocks,
                       void* out, hipStream_t stream) {
  // no more workgroups than fit at once: a partial second round of
  // workgroups would start late (the per-block-scale variant at B = 128
  // fits 7 per CU, not 8: 11.4 against 10.8 us before this cap)
  static std::atomic<int> caps[kMaxDevices];
  const int cap = per_device(caps, [] {
    const int cus = device_cu_count();
    return std::min(resident_grid(decompress_kernel<B, SBLK>, kThreads), (cus > 0 ? cus : 256) * kDecompressWgsPerCu<B>);
  });
  const int g = std::min<int>(tile_grid(nblocks), cap);
  hipLaunchKernelGGL((decompress_kernel<B, SBLK>), dim3(g), dim3(kThreads), 0,
                     stream, reinterpret_cast<const uint4*>(q), alpha, scale, nblocks, static_cast<uint4*>(out));
}

template <int B, int P>
void launch_decompress_sum_p(const Parts& parts, int64_t nblocks, void* out, hipStream_t stream) {
  hipLaunchKernelGGL((decompress_sum_kernel<B, P>), dim3(tile_grid(nblocks)), dim3(kThreads), 0,
                     stream, parts, nblocks, static_cast<uint4*>(out));
}

template <int B>
void launch_decompress_sum(const Parts& parts, int nparts, int64_t nblocks, void* out,
                           hipStream_t stream) {
  switch (nparts) {
    case 1: launch_decompress_sum_p<B, 1>(parts, nblocks, out, stream); break;
    case 2: launch_decompress_sum_p<B, 2>(parts, nblocks, out, stream); break;
    case 3: launch_decompress_sum_p<B, 3>(parts, nblocks, out, stream); break;
    case 4: launch_decompress_sum_p<B, 4>(parts, nblocks, out, stream); break;
    case 5: launch_decompress_sum_p<B, 5>(parts, nblocks, out, stream); break;
    case 6: launch_decompress_sum_p<B, 6>(parts, nblocks, out, stream); break;
    case 7: launch_decompress_sum_p<B, 7>(parts, nblocks, out, stream); break;
    default: launch_decompress_sum_p<B, 8>(parts, nblocks, out, stream); break;
  }
}

// Bytes of the compress workspace proper (barrier lines and partial maxima),
// rounded up so that the decompress-sum-compress intermediate after it is
// 256-byte aligned.
constexpr size_t kCompressWorkspace = (kSlotOffset + static_cast<size_t>(kSlotStride) * kMaxSlots + 255) / 256 * 256;

// One workgroup per CU at most (as the compress): at B = 64 one tile per
// wavefront on two workgroups per CU measured slower than two tiles per
// wavefront on one ([4096, 1600], 4 parts: 15.0 against 13.9-14.2 us).
template <int B, int TPW, int WAVES, int NP>
bool try_decompress_sum_compress_np(const Parts& parts, int64_t nblocks, float sqrt_eb, float* alpha,
                                    float* scale, char* ws, uint4* q, hipStream_t stream, unsigned polls) {
  static std::atomic<int> caps[kMaxDevices];
  const int cap = per_device(caps, [] {
    return fused_grid_cap(resident_grid(decompress_sum_compress_kernel<B, TPW, WAVES, NP>, 64 * WAVES));
  });
  const int64_t tiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int64_t g = ((tiles + TPW - 1) / TPW + WAVES - 1) / WAVES;
  if (g > cap) return false;
  hipLaunchKernelGGL((decompress_sum_compress_kernel<B, TPW, WAVES, NP>), dim3(g), dim3(64 * WAVES), 0,
                     stream, parts, nblocks, sqrt_eb, alpha, scale, ws, q, polls);
  return true;
}

template <int B, int TPW, int WAVES>
bool try_decompress_sum_compress(const Parts& parts, int nparts, int64_t nblocks, float sqrt_eb,
                                 float* alpha, float* scale, char* ws, uint4* q, hipStream_t stream,
                                 unsigned polls) {
  switch (nparts) {
    case 1: return try_decompress_sum_compress_np<B, TPW, WAVES, 1>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 2: return try_decompress_sum_compress_np<B, TPW, WAVES, 2>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 3: return try_decompress_sum_compress_np<B, TPW, WAVES, 3>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 4: return try_decompress_sum_compress_np<B, TPW, WAVES, 4>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 5: return try_decompress_sum_compress_np<B, TPW, WAVES, 5>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 6: return try_decompress_sum_compress_np<B, TPW, WAVES, 6>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    case 7: return try_decompress_sum_compress_np<B, TPW, WAVES, 7>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
    default: return try_decompress_sum_compress_np<B, TPW, WAVES, 8>(parts, nblocks, sqrt_eb, alpha, scale, ws, q, stream, polls);
  }
}

// Fused when the reduced tensor fits on chip (fewest tiles per wavefront
// first); otherwise the bf16 sum goes through the workspace and is compressed
// as any other tensor.
template <int B>
void launch_decompress_sum_compress(const Parts& parts, int nparts, int64_t nblocks, float energy,
                                    uint8_t* q, float* alpha, float* scale, void* workspace,
                                    hipStream_t stream, bool single_pass, unsigned polls) {
  const float sqrt_eb = static_cast<float>(sqrt(static_cast<double>(energy) * B));
  char* ws = static_cast<char*>(workspace);
  uint4* qv = reinterpret_cast<uint4*>(q);
  // 16 wavefronts per CU (128 VGPRs each) up to B = 128; at B = 256 the
  // rotation of the sum needs more registers, so 8 wavefronts (256 VGPRs),
  // two tiles each.  As in the compress, small tensors take workgroups of 4
  // or 8 wavefronts first, over more CUs: cold, 4 parts, [1024, 4096] at
  // B = 128 12.2 -> 10.4 us, [256, 1024] at B = 64 7.5 -> 5.6 us.
  if (single_pass) {
    if constexpr (B <= 128) {
      if (try_decompress_sum_compress<B, 1, kWavesC / 4>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
      if (try_decompress_sum_compress<B, 1, kWavesC / 2>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
      if (try_decompress_sum_compress<B, 1, kWavesC>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
      if (try_decompress_sum_compress<B, 2, kWavesC>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
    } else {
      if (try_decompress_sum_compress<B, 2, kWavesC / 2>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
    }
    if constexpr (B == 64)
      if (try_decompress_sum_compress<B, 4, kWavesC>(parts, nparts, nblocks, sqrt_eb, alpha, scale, ws, qv, stream, polls)) return;
  }
  void* sum = ws + kCompressWorkspace;
  launch_decompress_sum<B>(parts, nparts, nblocks, sum, stream);
  launch_compress<B>(sum, nblocks, energy, q, alpha, scale, workspace, stream, single_pass, polls);
}

template <int B, int MODE>
void launch_compress_streaming(const void* x, int64_t nblocks, float energy, const float* amax_prev,
                               uint8_t* q, float* alpha, float* scale, float* amax_out,
                               hipStream_t stream) {
  constexpr int W = MODE == kDsDelayed ? 8 : kWaves;
  const float sqrt_eb = static_cast<float>(sqrt(static_cast<double>(energy) * B));
  const int64_t tiles = (nblocks + kTileBlocks - 1) / kTileBlocks;
  const int g = static_cast<int>(std::min<int64_t>((tiles + W - 1) / W, INT32_MAX));
  hipLaunchKernelGGL((compress_streaming_kernel<B, MODE, W>), dim3(g), dim3(64 * W), 0,
                     stream, static_cast<const uint4*>(x), nblocks, sqrt_eb, amax_prev, alpha, scale,
                     reinterpret_cast<unsigned*>(amax_out), reinterpret_cast<uint4*>(q));
}

// Workgroups of the INT8 streaming kernels (kInt8Unroll pieces per thread per
// trip), at most cap.
int int8_grid(int64_t n16, int64_t cap) {
  const int64_t per = static_cast<int64_t>(kThreads) * kInt8Unroll;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((n16 + per - 1) / per, cap)));
}

taco_status_t check_shape_int8(int64_t tokens, int64_t hidden, int32_t block) {
  if (block != 0) return check_shape(tokens, hidden, block);
  if (tokens < 1 || hidden < 1 || hidden % 8 != 0) return TACO_ERR_SHAPE;
  if (tokens > (int64_t(1) << 40) / hidden) return TACO_ERR_SHAPE;
  return TACO_OK;
}

void launch_compress_int8(const void* x, int64_t n16, int32_t block, int8_t* q, float* scale,
                          void* workspace, hipStream_t stream) {
  const uint4* xv = static_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(q);
  const int g = int8_grid(n16, INT32_MAX);
  switch (block) {
    case 0: {
      float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + kPartialOffset);
      const int g1 = int8_grid(n16, kMaxPartials);
      hipLaunchKernelGGL(int8_absmax_kernel, dim3(g1), dim3(kThreads), 0, stream, xv, n16, partial);
      hipLaunchKernelGGL(int8_quant_tensor_kernel, dim3(g), dim3(kThreads), 0, stream, xv, n16, partial, g1,
                         scale, qv);
      break;
    }
    case 64: hipLaunchKernelGGL(int8_quant_block_kernel<8>, dim3(g), dim3(kThreads), 0, stream, xv, n16, scale, qv); break;
    case 128: hipLaunchKernelGGL(int8_quant_block_kernel<16>, dim3(g), dim3(kThreads), 0, stream, xv, n16, scale, qv); break;
    default: hipLaunchKernelGGL(int8_quant_block_kernel<32>, dim3(g), dim3(kThreads), 0, stream, xv, n16, scale, qv); break;
  }
}

void launch_decompress_int8(const int8_t* q, const float* scale, int64_t n16, int32_t block, void* out,
                            hipStream_t stream) {
  const uint2* qv = reinterpret_cast<const uint2*>(q);
  uint4* ov = static_cast<uint4*>(out);
  const int g = int8_grid(n16, INT32_MAX);
  switch (block) {
    case 0: hipLaunchKernelGGL(int8_dequant_kernel<0>, dim3(g), dim3(kThreads), 0, stream, qv, scale, n16, ov); break;
    case 64: hipLaunchKernelGGL(int8_dequant_kernel<8>, dim3(g), dim3(kThreads), 0, stream, qv, scale, n16, ov); break;
    case 128: hipLaunchKernelGGL(int8_dequant_kernel<16>, dim3(g), dim3(kThreads), 0, stream, qv, scale, n16, ov); break;
    default: hipLaunchKernelGGL(int8_dequant_kernel<32>, dim3(g), dim3(kThreads), 0, stream, qv, scale, n16, ov); break;
  }
}

// A byte range of a caller's buffer, for the aliasing checks.
struct Span {
  const void* p;
  size_t n;
};

bool overlap(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Whether an output overlaps another output or an input (inputs may overlap
// each other: they are only read).
bool aliased(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto i = outs.begin(); i != outs.end(); ++i) {
    for (auto j = i + 1; j != outs.end(); ++j)
      if (overlap(*i, *j)) return true;
    for (const Span& in : ins)
      if (overlap(*i, in)) return true;
  }
  return false;
}

bool parts_overlap(const Span& out, const Parts& parts, int nparts, size_t qn, size_t an) {
  for (int p = 0; p < nparts; ++p)
    if (overlap(out, {parts.q[p], qn}) || overlap(out, {parts.alpha[p], an}) || overlap(out, {parts.scale[p], 4}))
      return true;
  return false;
}

bool energy_ok(float e) { return e >= kMinEnergy && e <= kMaxEnergy; }

taco_status_t check_flags(uint32_t flags) {
  return (flags & ~static_cast<uint32_t>(TACO_FLAG_TWO_PASS)) == 0 ? TACO_OK : TACO_ERR_FLAGS;
}

}  // namespace

// Workspace of taco_compress_noalloc: the compress workspace (barrier state
// and partial maxima) in device memory the library holds itself, one copy per
// GPU until the process ends.  Static storage starts zeroed, and every call
// leaves the barrier state ready for the next one, so nothing clears it.  In
// host code the name stands for no device address: the kernels get the
// address hipGetSymbolAddress returns on each device.
static __device__ __align__(256) char scratch[kCompressWorkspace];

namespace {

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up once per device), or null
// if the lookup fails.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

// ----------------------------------------------------------------- C ABI

extern "C" {

const char* taco_status_string(taco_status_t status) {
  switch (status) {
    case TACO_OK: return "TACO_OK";
    case TACO_ERR_NULL: return "TACO_ERR_NULL: a required pointer is NULL";
    case TACO_ERR_ALIGN: return "TACO_ERR_ALIGN: a pointer is not aligned as required";
    case TACO_ERR_SHAPE: return "TACO_ERR_SHAPE: tokens/hidden invalid or hidden % block != 0";
    case TACO_ERR_UNSUPPORTED_BLOCK: return "TACO_ERR_UNSUPPORTED_BLOCK: block must be 64, 128 or 256";
    case TACO_ERR_BAD_ENERGY: return "TACO_ERR_BAD_ENERGY: target energy must be finite, in [2^-40, 2^40]";
    case TACO_ERR_WORKSPACE: return "TACO_ERR_WORKSPACE: workspace too small";
    case TACO_ERR_BAD_NPARTS: return "TACO_ERR_BAD_NPARTS: nparts must be in [1, 8]";
    case TACO_ERR_HIP: return "TACO_ERR_HIP: a HIP call or kernel launch failed";
    case TACO_ERR_FLAGS: return "TACO_ERR_FLAGS: unknown bit in flags";
    case TACO_ERR_ALIAS: return "TACO_ERR_ALIAS: an output buffer overlaps an input or another output";
  }
  return "TACO_ERR_UNKNOWN";
}

const char* taco_version(void) { return "0.4.0"; }

int taco_compress_is_single_pass(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK || device_cu_count() <= 0) return -1;
  const int64_t nblocks = tokens * (hidden / block);
  bool fits;
  switch (block) {
    case 64: fits = launch_fused<64>(nullptr, nblocks, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr, false, 0); break;
    case 128: fits = launch_fused<128>(nullptr, nblocks, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr, false, 0); break;
    default: fits = launch_fused<256>(nullptr, nblocks, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr, false, 0); break;
  }
  return fits ? 1 : 0;
}

taco_status_t taco_workspace_timed_out(const void* workspace, taco_stream_t stream, int* timed_out) {
  if (workspace == nullptr || timed_out == nullptr) return TACO_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return TACO_ERR_ALIGN;
  unsigned flag = 0;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const char* root = static_cast<const char*>(workspace) + offsetof(RootLine, timed_out);
  if (hipMemcpyAsync(&flag, root, sizeof(flag), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return TACO_ERR_HIP;
  *timed_out = flag != 0 ? 1 : 0;
  return TACO_OK;
}

int64_t taco_num_scales(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK) return -1;
  return tokens * (hidden / block);
}

size_t taco_compress_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK) return 0;
  return kCompressWorkspace;   // leaf lines, partial maxima and barrier slots
}

taco_status_t taco_compress_ex(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                               float target_energy, uint8_t* q_fp8, float* alpha, float* scale,
                               void* workspace, size_t workspace_bytes, uint32_t flags,
                               uint32_t barrier_polls, taco_stream_t stream) {
  if (!x_bf16 || !q_fp8 || !alpha || !scale || !workspace) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(x_bf16, 16) || !aligned(q_fp8, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      !aligned(workspace, 256))
    return TACO_ERR_ALIGN;
  if (!energy_ok(target_energy)) return TACO_ERR_BAD_ENERGY;
  if (workspace_bytes < taco_compress_workspace_bytes(tokens, hidden, block)) return TACO_ERR_WORKSPACE;
  if (check_flags(flags) != TACO_OK) return TACO_ERR_FLAGS;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  if (aliased({{q_fp8, n}, {alpha, 4 * static_cast<size_t>(nblocks)}, {scale, 4}, {workspace, workspace_bytes}},
              {{x_bf16, 2 * n}}))
    return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool single = (flags & TACO_FLAG_TWO_PASS) == 0;
  const unsigned polls = barrier_polls == 0 ? kDefaultSpinLimit : barrier_polls;
  switch (block) {
    case 64: launch_compress<64>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, workspace, s, single, polls); break;
    case 128: launch_compress<128>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, workspace, s, single, polls); break;
    default: launch_compress<256>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, workspace, s, single, polls); break;
  }
  return launched();
}

taco_status_t taco_compress(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                            float target_energy, uint8_t* q_fp8, float* alpha, float* scale,
                            void* workspace, size_t workspace_bytes, taco_stream_t stream) {
  return taco_compress_ex(x_bf16, tokens, hidden, block, target_energy, q_fp8, alpha, scale, workspace,
                          workspace_bytes, 0, 0, stream);
}

taco_status_t taco_compress_noalloc(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                                    float target_energy, uint8_t* q_fp8, float* alpha, float* scale,
                                    uint32_t flags, uint32_t barrier_polls, taco_stream_t stream) {
  if (!x_bf16 || !q_fp8 || !alpha || !scale) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (taco_compress_workspace_bytes(tokens, hidden, block) > sizeof(scratch)) return TACO_ERR_WORKSPACE;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return TACO_ERR_HIP;
  return taco_compress_ex(x_bf16, tokens, hidden, block, target_energy, q_fp8, alpha, scale, ws,
                          sizeof(scratch), flags, barrier_polls, stream);
}

taco_status_t taco_decompress(const uint8_t* q_fp8, const float* alpha, const float* scale,
                              int64_t tokens, int64_t hidden, int32_t block, void* y_bf16,
                              taco_stream_t stream) {
  if (!q_fp8 || !alpha || !scale || !y_bf16) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(q_fp8, 16) || !aligned(y_bf16, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
    return TACO_ERR_ALIGN;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  if (aliased({{y_bf16, 2 * n}}, {{q_fp8, n}, {alpha, 4 * static_cast<size_t>(nblocks)}, {scale, 4}}))
    return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_decompress<64, false>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
    case 128: launch_decompress<128, false>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
    default: launch_decompress<256, false>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
  }
  return launched();
}

taco_status_t taco_decompress_sum(const uint8_t* const* q_fp8, const float* const* alpha,
                                  const float* const* scale, int32_t nparts, int64_t tokens,
                                  int64_t hidden, int32_t block, void* out_bf16,
                                  taco_stream_t stream) {
  if (!q_fp8 || !alpha || !scale || !out_bf16) return TACO_ERR_NULL;
  if (nparts < 1 || nparts > TACO_MAX_PARTS) return TACO_ERR_BAD_NPARTS;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  Parts parts{};
  for (int p = 0; p < nparts; ++p) {
    if (!q_fp8[p] || !alpha[p] || !scale[p]) return TACO_ERR_NULL;
    if (!aligned(q_fp8[p], 16) || !aligned(alpha[p], 4) || !aligned(scale[p], 4)) return TACO_ERR_ALIGN;
    parts.q[p] = reinterpret_cast<const uint4*>(q_fp8[p]);
    parts.alpha[p] = alpha[p];
    parts.scale[p] = scale[p];
  }
  if (!aligned(out_bf16, 16)) return TACO_ERR_ALIGN;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  if (parts_overlap({out_bf16, 2 * n}, parts, nparts, n, 4 * static_cast<size_t>(nblocks))) return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_decompress_sum<64>(parts, nparts, nblocks, out_bf16, s); break;
    case 128: launch_decompress_sum<128>(parts, nparts, nblocks, out_bf16, s); break;
    default: launch_decompress_sum<256>(parts, nparts, nblocks, out_bf16, s); break;
  }
  return launched();
}

size_t taco_compress_int8_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape_int8(tokens, hidden, block) != TACO_OK) return 0;
  return block == 0 ? kCompressWorkspace : 0;
}

taco_status_t taco_compress_int8(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                                 int8_t* q_int8, float* scale, void* workspace, size_t workspace_bytes,
                                 taco_stream_t stream) {
  if (!x_bf16 || !q_int8 || !scale || (block == 0 && !workspace)) return TACO_ERR_NULL;
  const taco_status_t st = check_shape_int8(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(x_bf16, 16) || !aligned(q_int8, 16) || !aligned(scale, 4) ||
      (block == 0 && !aligned(workspace, 256)))
    return TACO_ERR_ALIGN;
  if (block == 0 && workspace_bytes < kCompressWorkspace) return TACO_ERR_WORKSPACE;
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  const size_t sbytes = block == 0 ? 4 : 4 * (n / static_cast<size_t>(block));
  if (aliased({{q_int8, n}, {scale, sbytes}, {block == 0 ? workspace : nullptr, workspace_bytes}}, {{x_bf16, 2 * n}}))
    return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  launch_compress_int8(x_bf16, tokens * hidden / 8, block, q_int8, scale, workspace,
                       reinterpret_cast<hipStream_t>(stream));
  return launched();
}

taco_status_t taco_decompress_int8(const int8_t* q_int8, const float* scale, int64_t tokens, int64_t hidden,
                                   int32_t block, void* y_bf16, taco_stream_t stream) {
  if (!q_int8 || !scale || !y_bf16) return TACO_ERR_NULL;
  const taco_status_t st = check_shape_int8(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(q_int8, 16) || !aligned(y_bf16, 16) || !aligned(scale, 4)) return TACO_ERR_ALIGN;
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  const size_t sbytes = block == 0 ? 4 : 4 * (n / static_cast<size_t>(block));
  if (aliased({{y_bf16, 2 * n}}, {{q_int8, n}, {scale, sbytes}})) return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  launch_decompress_int8(q_int8, scale, tokens * hidden / 8, block, y_bf16, reinterpret_cast<hipStream_t>(stream));
  return launched();
}

size_t taco_decompress_sum_compress_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK) return 0;
  return kCompressWorkspace + static_cast<size_t>(tokens) * static_cast<size_t>(hidden) * 2;
}

taco_status_t taco_decompress_sum_compress_ex(const uint8_t* const* q_fp8, const float* const* alpha,
                                              const float* const* scale, int32_t nparts, int64_t tokens,
                                              int64_t hidden, int32_t block, float target_energy,
                                              uint8_t* q_out, float* alpha_out, float* scale_out,
                                              void* workspace, size_t workspace_bytes, uint32_t flags,
                                              uint32_t barrier_polls, taco_stream_t stream) {
  if (!q_fp8 || !alpha || !scale || !q_out || !alpha_out || !scale_out || !workspace) return TACO_ERR_NULL;
  if (nparts < 1 || nparts > TACO_MAX_PARTS) return TACO_ERR_BAD_NPARTS;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!energy_ok(target_energy)) return TACO_ERR_BAD_ENERGY;
  Parts parts{};
  for (int p = 0; p < nparts; ++p) {
    if (!q_fp8[p] || !alpha[p] || !scale[p]) return TACO_ERR_NULL;
    if (!aligned(q_fp8[p], 16) || !aligned(alpha[p], 4) || !aligned(scale[p], 4)) return TACO_ERR_ALIGN;
    parts.q[p] = reinterpret_cast<const uint4*>(q_fp8[p]);
    parts.alpha[p] = alpha[p];
    parts.scale[p] = scale[p];
  }
  if (!aligned(q_out, 16) || !aligned(alpha_out, 4) || !aligned(scale_out, 4) || !aligned(workspace, 256))
    return TACO_ERR_ALIGN;
  if (workspace_bytes < taco_decompress_sum_compress_workspace_bytes(tokens, hidden, block))
    return TACO_ERR_WORKSPACE;
  if (check_flags(flags) != TACO_OK) return TACO_ERR_FLAGS;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  const size_t an = 4 * static_cast<size_t>(nblocks);
  const Span outs[4] = {{q_out, n}, {alpha_out, an}, {scale_out, 4}, {workspace, workspace_bytes}};
  if (aliased({outs[0], outs[1], outs[2], outs[3]}, {}))
    return TACO_ERR_ALIAS;
  for (const Span& o : outs)
    if (parts_overlap(o, parts, nparts, n, an)) return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool single = (flags & TACO_FLAG_TWO_PASS) == 0;
  const unsigned polls = barrier_polls == 0 ? kDefaultSpinLimit : barrier_polls;
  switch (block) {
    case 64: launch_decompress_sum_compress<64>(parts, nparts, nblocks, target_energy, q_out, alpha_out, scale_out, workspace, s, single, polls); break;
    case 128: launch_decompress_sum_compress<128>(parts, nparts, nblocks, target_energy, q_out, alpha_out, scale_out, workspace, s, single, polls); break;
    default: launch_decompress_sum_compress<256>(parts, nparts, nblocks, target_energy, q_out, alpha_out, scale_out, workspace, s, single, polls); break;
  }
  return launched();
}

taco_status_t taco_decompress_sum_compress(const uint8_t* const* q_fp8, const float* const* alpha,
                                           const float* const* scale, int32_t nparts, int64_t tokens,
                                           int64_t hidden, int32_t block, float target_energy,
                                           uint8_t* q_out, float* alpha_out, float* scale_out,
                                           void* workspace, size_t workspace_bytes,
                                           taco_stream_t stream) {
  return taco_decompress_sum_compress_ex(q_fp8, alpha, scale, nparts, tokens, hidden, block, target_energy,
                                         q_out, alpha_out, scale_out, workspace, workspace_bytes, 0, 0,
                                         stream);
}

taco_status_t taco_compress_blockscale(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                                       float target_energy, uint8_t* q_fp8, float* alpha,
                                       float* scale_blk, taco_stream_t stream) {
  if (!x_bf16 || !q_fp8 || !alpha || !scale_blk) return TACO_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_fp8, 16) || !aligned(alpha, 4) || !aligned(scale_blk, 4))
    return TACO_ERR_ALIGN;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!energy_ok(target_energy)) return TACO_ERR_BAD_ENERGY;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  const size_t an = 4 * static_cast<size_t>(nblocks);
  if (aliased({{q_fp8, n}, {alpha, an}, {scale_blk, an}}, {{x_bf16, 2 * n}})) return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_compress_streaming<64, kDsBlockGuard>(x_bf16, nblocks, target_energy, nullptr, q_fp8, alpha, scale_blk, nullptr, s); break;
    case 128: launch_compress_streaming<128, kDsBlockGuard>(x_bf16, nblocks, target_energy, nullptr, q_fp8, alpha, scale_blk, nullptr, s); break;
    default: launch_compress_streaming<256, kDsBlockGuard>(x_bf16, nblocks, target_energy, nullptr, q_fp8, alpha, scale_blk, nullptr, s); break;
  }
  return launched();
}

taco_status_t taco_decompress_blockscale(const uint8_t* q_fp8, const float* alpha, const float* scale_blk,
                                         int64_t tokens, int64_t hidden, int32_t block, void* y_bf16,
                                         taco_stream_t stream) {
  if (!q_fp8 || !alpha || !scale_blk || !y_bf16) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(q_fp8, 16) || !aligned(y_bf16, 16) || !aligned(alpha, 4) || !aligned(scale_blk, 4))
    return TACO_ERR_ALIGN;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  const size_t an = 4 * static_cast<size_t>(nblocks);
  if (aliased({{y_bf16, 2 * n}}, {{q_fp8, n}, {alpha, an}, {scale_blk, an}})) return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_decompress<64, true>(q_fp8, alpha, scale_blk, nblocks, y_bf16, s); break;
    case 128: launch_decompress<128, true>(q_fp8, alpha, scale_blk, nblocks, y_bf16, s); break;
    default: launch_decompress<256, true>(q_fp8, alpha, scale_blk, nblocks, y_bf16, s); break;
  }
  return launched();
}

taco_status_t taco_compress_delayed(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                                    float target_energy, const float* amax_prev, uint8_t* q_fp8,
                                    float* alpha, float* scale, float* amax_out, taco_stream_t stream) {
  if (!x_bf16 || !amax_prev || !q_fp8 || !alpha || !scale || !amax_out) return TACO_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_fp8, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      !aligned(amax_prev, 4) || !aligned(amax_out, 4))
    return TACO_ERR_ALIGN;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!energy_ok(target_energy)) return TACO_ERR_BAD_ENERGY;
  const int64_t nblocks = tokens * (hidden / block);
  const size_t n = static_cast<size_t>(tokens) * static_cast<size_t>(hidden);
  constexpr size_t kAmaxBytes = 4 * TACO_AMAX_FLOATS;
  if (aliased({{q_fp8, n}, {alpha, 4 * static_cast<size_t>(nblocks)}, {scale, 4}, {amax_out, kAmaxBytes}},
              {{x_bf16, 2 * n}, {amax_prev, kAmaxBytes}}))
    return TACO_ERR_ALIAS;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_compress_streaming<64, kDsDelayed>(x_bf16, nblocks, target_energy, amax_prev, q_fp8, alpha, scale, amax_out, s); break;
    case 128: launch_compress_streaming<128, kDsDelayed>(x_bf16, nblocks, target_energy, amax_prev, q_fp8, alpha, scale, amax_out, s); break;
    default: launch_compress_streaming<256, kDsDelayed>(x_bf16, nblocks, target_energy, amax_prev, q_fp8, alpha, scale, amax_out, s); break;
  }
  return launched();
}

}  // extern "C"
