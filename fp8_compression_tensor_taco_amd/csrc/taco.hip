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
// Work decomposition ("quad layout").  Four consecutive lanes of a wavefront
// (a quad) own one B-element block; lane q of the quad holds the elements
// 32*a + 8*q + b of the block, a = 0 .. B/32-1 and b = 0..7, i.e. B/32 "chunks"
// of 8 consecutive elements (16 bytes of bf16, 8 bytes of FP8).  A wavefront
// therefore covers 16 blocks, and per load instruction the four lanes of a quad
// read 64 contiguous bytes of bf16.  With this layout the Walsh-Hadamard
// butterflies on element-index bits 0-2 and 5.. are in-lane register
// operations and only bits 3 and 4 cross lanes, both inside the quad, where a
// DPP quad permutation reaches the partner lane without LDS traffic.
//
// The cross-lane butterfly is computed as v + c*partner with a per-lane sign
// c = +-1: lanes whose index bit is clear get a+b, the others get a-b, which is
// the negated (b-a) they should hold.  The negation is tracked instead of
// undone: after both quad stages lane q holds its outputs times
// D(q) = c1(q)*c2(q), and D is folded into the scale applied next.
//
// Compression needs the tensor-wide max|y| before any code can be written, so
// it runs as two kernels: a statistics pass (energy, alpha, rotation,
// per-workgroup max) and a quantisation pass that re-reads x (the second read
// of a tensor of this size is largely served by the Infinity Cache), folds the
// workgroup maxima into s and writes the codes.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "taco.h"

namespace {

constexpr int kThreads = 256;        // 4 wavefronts per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kBlocksPerWave = 16;   // one block per quad
constexpr float kQmax = 448.0f;      // largest E4M3FN magnitude
constexpr int kMaxPartials = 4096;   // workgroups of the statistics pass
constexpr int kWgPerCu = 8;

constexpr int kQuadXor1 = 0xB1;      // DPP quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // DPP quad_perm [2,3,0,1]

template <int B>
struct Blk {
  static constexpr int NA = B / 32;               // 8-element chunks per lane
  static constexpr int C16 = B / 8;               // 16-byte bf16 chunks per block
  static constexpr float inv_b = 1.0f / B;        // exact (power of two)
  static constexpr float rsqrt_b = B == 64 ? 0.125f
                                 : B == 128 ? 0.0883883476483184405f  // fp32(1/sqrt(128))
                                            : 0.0625f;
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- helpers

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

// bf16 -> fp32 fused with the first butterfly (index bit 0): for each packed
// pair (x0, x1) the dot products with (1, 1) and (1, -1) give x0+x1 and x0-x1.
__device__ __forceinline__ void widen_bf16x8_stage0(const uint4 u, float (&v)[8]) {
  constexpr unsigned kPlusPlus = 0x3F803F80u, kPlusMinus = 0xBF803F80u;
  v[0] = dot2_bf16(u.x, kPlusPlus, 0.0f); v[1] = dot2_bf16(u.x, kPlusMinus, 0.0f);
  v[2] = dot2_bf16(u.y, kPlusPlus, 0.0f); v[3] = dot2_bf16(u.y, kPlusMinus, 0.0f);
  v[4] = dot2_bf16(u.z, kPlusPlus, 0.0f); v[5] = dot2_bf16(u.z, kPlusMinus, 0.0f);
  v[6] = dot2_bf16(u.w, kPlusPlus, 0.0f); v[7] = dot2_bf16(u.w, kPlusMinus, 0.0f);
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

// Butterflies across the lane's chunks (index bits 5 ..).
template <int NA>
__device__ __forceinline__ void fwht_across_chunks(float (&v)[NA][8]) {
#pragma unroll
  for (int h = 1; h < NA; h <<= 1) {
#pragma unroll
    for (int a = 0; a < NA; a += 2 * h) {
#pragma unroll
      for (int c = a; c < a + h; ++c) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = v[c][j], y = v[c + h][j];
          v[c][j] = x + y;
          v[c + h][j] = x - y;
        }
      }
    }
  }
}

// Butterflies on index bits 3 and 4 (across the quad), with the sign debt
// described above; c1 = +-1 by quad-lane bit 0, c2 by quad-lane bit 1.
template <int NA>
__device__ __forceinline__ void fwht_across_quad(float (&v)[NA][8], float c1, float c2) {
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[a][j] = fmaf(dpp<kQuadXor1>(v[a][j]), c1, v[a][j]);
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[a][j] = fmaf(dpp<kQuadXor2>(v[a][j]), c2, v[a][j]);
}

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<kQuadXor1>(v);
  return v + dpp<kQuadXor2>(v);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Max over the workgroup; every thread gets the result.
__device__ __forceinline__ float workgroup_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
  return m;
}

// ASH scale from the block's sum of squares: sqrt(E / m), m = ss / B; 1 if zero.
template <int B>
__device__ __forceinline__ float ash_scale(float ss, float energy) {
  return ss > 0.0f ? sqrtf(energy / (ss * Blk<B>::inv_b)) : 1.0f;
}

// 8 values * c -> 8 E4M3FN codes (native gfx950 conversion, round to nearest
// even).  |v*c| never exceeds 448 by more than a few ulps, which rounds to 448.
__device__ __forceinline__ uint2 to_fp8x8(const float (&v)[8], float c) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0] * c, v[1] * c, 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2] * c, v[3] * c, lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4] * c, v[5] * c, 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6] * c, v[7] * c, hi, true);
  return make_uint2(static_cast<unsigned>(lo), static_cast<unsigned>(hi));
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

// Lane geometry inside a wavefront tile of 16 blocks.
struct Lane {
  int quad;       // block of the tile owned by this lane's quad (0..15)
  int ql;         // position in the quad (0..3)
  float c1, c2;   // butterfly signs for the two quad stages
  float debt;     // c1*c2: sign the quad stages leave on this lane's outputs
  __device__ __forceinline__ Lane() {
    const int lane = threadIdx.x & 63;
    quad = lane >> 2;
    ql = lane & 3;
    c1 = (ql & 1) ? -1.0f : 1.0f;
    c2 = (ql & 2) ? -1.0f : 1.0f;
    debt = c1 * c2;
  }
};

// ----------------------------------------------------------------- kernels
//
// Every kernel walks 16-block tiles with a wavefront-uniform grid-stride loop
// that keeps U tiles' loads in flight per lane.  Quads whose block lies past
// the end compute on zeros and store nothing.

// Load a tile's bf16 chunks for this lane and return the full Hadamard
// transform of its block (times the lane's sign debt), plus the block's
// sum of squares (identical in the four lanes of the quad).
template <int B>
__device__ __forceinline__ float rotate_bf16(const uint4 (&raw)[Blk<B>::NA], float (&v)[Blk<B>::NA][8],
                                             const Lane& ln) {
  constexpr int NA = Blk<B>::NA;
  const float ss = quad_sum(sum_squares_bf16<NA>(raw));
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    widen_bf16x8_stage0(raw[a], v[a]);
    fwht_chunk<2>(v[a]);
  }
  fwht_across_chunks<NA>(v);
  fwht_across_quad<NA>(v, ln.c1, ln.c2);
  return ss;
}

// Compress, statistics pass: alpha for every block, and per workgroup the max
// over its blocks of alpha_k * max|H x_k| / sqrt(B).
template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_stats_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float energy,
    float* __restrict__ alpha, float* __restrict__ partial) {
  constexpr int NA = Blk<B>::NA;
  __shared__ float red[kWaves];
  const Lane ln;
  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  float amax = 0.0f;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    uint4 raw[U][NA];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
      for (int a = 0; a < NA; ++a)
        raw[u][a] = ok ? x[k * Blk<B>::C16 + 4 * a + ln.ql] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      float v[NA][8];
      const float a = ash_scale<B>(rotate_bf16<B>(raw[u], v, ln), energy);
      if (ok && ln.ql == 0) alpha[k] = a;
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < NA; ++c)
#pragma unroll
        for (int j = 0; j < 8; j += 2) m = fmaxf(fmaxf(m, fabsf(v[c][j])), fabsf(v[c][j + 1]));
      amax = fmaxf(amax, m * (a * Blk<B>::rsqrt_b));
    }
  }
  const float wg = workgroup_max(amax, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = wg;
}

// Compress, quantisation pass: s from the workgroup maxima, then codes.
template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_quant_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float energy,
    const float* __restrict__ partial, int npartial, float* __restrict__ scale,
    uint2* __restrict__ q) {
  constexpr int NA = Blk<B>::NA;
  __shared__ float red[kWaves];
  const Lane ln;
  float A = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += kThreads) A = fmaxf(A, partial[i]);
  A = workgroup_max(A, red);
  const float s = A > 0.0f ? kQmax / A : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;

  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    uint4 raw[U][NA];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
      for (int a = 0; a < NA; ++a)
        raw[u][a] = ok ? x[k * Blk<B>::C16 + 4 * a + ln.ql] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      float v[NA][8];
      const float a = ash_scale<B>(rotate_bf16<B>(raw[u], v, ln), energy);
      const float c = ((a * s) * Blk<B>::rsqrt_b) * ln.debt;
#pragma unroll
      for (int ch = 0; ch < NA; ++ch) {
        const uint2 codes = to_fp8x8(v[ch], c);
        if (ok) q[k * Blk<B>::C16 + 4 * ch + ln.ql] = codes;
      }
    }
  }
}

// ----------------------------------------------------------------- MFMA path
//
// The rotation of raw x is a dense contraction y = H_B x against a +-1 matrix,
// and raw x is exactly bf16, so it can run on the matrix cores with no loss:
// v_mfma_f32_16x16x32_bf16 multiplies exact bf16 operands and accumulates in
// fp32.  The product is formed transposed, C[m][n] = sum_k H[m][k] X[n][k],
// with the 16 columns n of the MFMA being 16 blocks (one wavefront tile):
//   B operand: lane (g, n), g = lane/16, holds 8 elements of block n,
//              element 32*kt + 8*g + s (s = 0..7) in K-step kt;
//   A operand: lane (g, r) holds H[16*mt + r][32*kt + 8*g + s];
//   C:         lane (g, n) receives y[block n][16*mt + 4*g + i], i = 0..3.
// Because H[i][j] = (-1)^popcount(i & j) factors over index bits, the A
// operand for M-tile mt and K-step kt is F_{mt&1} * (-1)^popcount((mt>>1) & kt)
// with two lane-dependent fragments
//   F_e[lane (g, r)][s] = (-1)^(popcount(r & s & 7) + (r>>3)*(g&1) + e*(g>>1)),
// so four constant register sets (F_0, F_1 and their negations) cover every
// (mt, kt) pair.  The element loads are the same 64-byte-per-block pattern as
// the quad layout; the per-block sum of squares is reduced over the 4 lanes of
// a column with two cross-row shuffles.

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

// Sum of squares of a column's block: the lane's 8*B/32 elements, then the
// 4 lanes (g = 0..3) of the column.  Every lane of the column gets the same sum.
template <int B>
__device__ __forceinline__ float column_sum_squares(const uint4 (&xr)[B / 32]) {
  float ss = sum_squares_bf16<B / 32>(xr);
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  return ss;
}

template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_stats_mfma_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float energy,
    float* __restrict__ alpha, float* __restrict__ partial) {
  constexpr int NK = B / 32, NM = B / 16;
  __shared__ float red[kWaves];
  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  float amax = 0.0f;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    uint4 xr[U][NK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + n;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
      for (int kt = 0; kt < NK; ++kt)
        xr[u][kt] = ok ? x[k * Blk<B>::C16 + 4 * kt + g] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + n;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      const float a = ash_scale<B>(column_sum_squares<B>(xr[u]), energy);
      if (ok && g == 0) alpha[k] = a;
      float m = 0.0f;
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const f32x4_t y = hadamard_mtile<B>(F, xr[u], mt);
        m = fmaxf(fmaxf(m, fabsf(y[0])), fabsf(y[1]));
        m = fmaxf(fmaxf(m, fabsf(y[2])), fabsf(y[3]));
      }
      amax = fmaxf(amax, m * (a * Blk<B>::rsqrt_b));
    }
  }
  const float wg = workgroup_max(amax, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = wg;
}

template <int B, int U>
__global__ __launch_bounds__(kThreads) void compress_quant_mfma_kernel(
    const uint4* __restrict__ x, int64_t nblocks, float energy,
    const float* __restrict__ partial, int npartial, float* __restrict__ scale,
    unsigned* __restrict__ q) {
  constexpr int NK = B / 32, NM = B / 16;
  __shared__ float red[kWaves];
  float A = 0.0f;
  for (int i = threadIdx.x; i < npartial; i += kThreads) A = fmaxf(A, partial[i]);
  A = workgroup_max(A, red);
  const float s = A > 0.0f ? kQmax / A : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;

  const HadFrag F = make_hadamard_fragments();
  const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    uint4 xr[U][NK];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + n;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
      for (int kt = 0; kt < NK; ++kt)
        xr[u][kt] = ok ? x[k * Blk<B>::C16 + 4 * kt + g] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + n;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      const float a = ash_scale<B>(column_sum_squares<B>(xr[u]), energy);
      const float c = (a * s) * Blk<B>::rsqrt_b;
#pragma unroll
      for (int mt = 0; mt < NM; ++mt) {
        const f32x4_t y = hadamard_mtile<B>(F, xr[u], mt);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] * c, y[1] * c, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] * c, y[3] * c, w, true);
        if (ok) q[k * (B / 4) + 4 * mt + g] = static_cast<unsigned>(w);
      }
    }
  }
}

// Hadamard transform of one lane's decoded chunks (bits 0-2, 5.., then 3-4).
template <int NA>
__device__ __forceinline__ void rotate_f32(float (&v)[NA][8], const Lane& ln) {
#pragma unroll
  for (int a = 0; a < NA; ++a) fwht_chunk<1>(v[a]);
  fwht_across_chunks<NA>(v);
  fwht_across_quad<NA>(v, ln.c1, ln.c2);
}

// Decompress: decode, rotate, multiply by 1/(alpha_k s sqrt(B)), round to bf16.
template <int B, int U>
__global__ __launch_bounds__(kThreads) void decompress_kernel(
    const uint2* __restrict__ q, const float* __restrict__ alpha,
    const float* __restrict__ scale, int64_t nblocks, uint4* __restrict__ out) {
  constexpr int NA = Blk<B>::NA;
  const Lane ln;
  const float s = *scale;
  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    uint2 raw[U][NA];
    float al[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
      for (int a = 0; a < NA; ++a)
        raw[u][a] = ok ? q[k * Blk<B>::C16 + 4 * a + ln.ql] : make_uint2(0, 0);
      al[u] = ok ? alpha[k] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      float v[NA][8];
#pragma unroll
      for (int a = 0; a < NA; ++a) from_fp8x8(raw[u][a], v[a]);
      rotate_f32<NA>(v, ln);
      const float r = (Blk<B>::rsqrt_b / (al[u] * s)) * ln.debt;
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const uint4 o = to_bf16x8(v[a], r);
        if (ok) out[k * Blk<B>::C16 + 4 * a + ln.ql] = o;
      }
    }
  }
}

struct Parts {
  const uint2* q[TACO_MAX_PARTS];
  const float* alpha[TACO_MAX_PARTS];
  const float* scale[TACO_MAX_PARTS];
};

// Decompress-and-sum.  The rotation is linear, so the parts are combined
// before it: acc = sum_p decode(q_p) / (alpha_{p,k} s_p), then one rotation
// and the 1/sqrt(B) factor.  This is the same sum as decompressing each part
// and adding the results, with P-1 fewer transforms per block.
template <int B, int U>
__global__ __launch_bounds__(kThreads) void decompress_sum_kernel(
    Parts parts, int nparts, int64_t nblocks, uint4* __restrict__ out) {
  constexpr int NA = Blk<B>::NA;
  const Lane ln;
  float s[TACO_MAX_PARTS];
#pragma unroll
  for (int p = 0; p < TACO_MAX_PARTS; ++p) s[p] = p < nparts ? *parts.scale[p] : 1.0f;
  const int64_t ntiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t W = static_cast<int64_t>(gridDim.x) * kWaves;
  for (int64_t t0 = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6); t0 < ntiles;
       t0 += W * U) {
    float acc[U][NA][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[u][a][j] = 0.0f;
#pragma unroll
    for (int p = 0; p < TACO_MAX_PARTS; ++p) {
      if (p >= nparts) break;
      uint2 raw[U][NA];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
        const bool ok = (t0 + u * W < ntiles) && k < nblocks;
#pragma unroll
        for (int a = 0; a < NA; ++a)
          raw[u][a] = ok ? parts.q[p][k * Blk<B>::C16 + 4 * a + ln.ql] : make_uint2(0, 0);
        w[u] = ok ? parts.alpha[p][k] : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wt = 1.0f / (w[u] * s[p]);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          float d[8];
          from_fp8x8(raw[u][a], d);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[u][a][j] = fmaf(d[j], wt, acc[u][a][j]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = (t0 + u * W) * kBlocksPerWave + ln.quad;
      const bool ok = (t0 + u * W < ntiles) && k < nblocks;
      rotate_f32<NA>(acc[u], ln);
      const float r = Blk<B>::rsqrt_b * ln.debt;
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const uint4 o = to_bf16x8(acc[u][a], r);
        if (ok) out[k * Blk<B>::C16 + 4 * a + ln.ql] = o;
      }
    }
  }
}

// ----------------------------------------------------------------- host side

// Tiles (16 blocks, one wavefront) kept in flight per lane per loop trip.
template <int B> constexpr int unroll_compress() { return B == 256 ? 1 : B == 128 ? 2 : 4; }
template <int B> constexpr int unroll_decompress() { return B == 256 ? 2 : B == 128 ? 4 : 8; }
template <int B> constexpr int unroll_sum() { return B == 256 ? 1 : B == 128 ? 1 : 2; }

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  static int cached[64] = {0};
  if (dev < 0 || dev >= 64) return -1;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    cached[dev] = n;
  }
  return cached[dev];
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

// Workgroups for a grid-stride walk over 16-block tiles, U tiles per wavefront
// per trip, capped at `cap`.
int grid_for(int64_t nblocks, int unroll, int cap) {
  const int64_t tiles = (nblocks + kBlocksPerWave - 1) / kBlocksPerWave;
  const int64_t per_wg = static_cast<int64_t>(kWaves) * unroll;
  int64_t g = (tiles + per_wg - 1) / per_wg;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

int wg_cap() {
  const int cus = device_cu_count();
  return (cus > 0 ? cus : 256) * kWgPerCu;
}

// Workgroups of `kernel` that fit on the whole device at once (a persistent
// grid: every wavefront then walks several tiles and the last round has no
// partially filled machine).
template <typename Kernel>
int resident_grid(Kernel kernel) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int cus = device_cu_count();
  return per_cu * (cus > 0 ? cus : 256);
}

taco_status_t launched() { return hipGetLastError() == hipSuccess ? TACO_OK : TACO_ERR_HIP; }

int g_engine = TACO_ENGINE_AUTO;   // rotation engine of taco_compress (process-wide)

template <int B>
void launch_compress(const void* x, int64_t nblocks, float energy, uint8_t* q, float* alpha,
                     float* scale, float* partial, hipStream_t stream) {
  constexpr int U = unroll_compress<B>();
  const bool mfma = g_engine != TACO_ENGINE_VALU;
  auto stats = mfma ? compress_stats_mfma_kernel<B, U> : compress_stats_kernel<B, U>;
  static const int cap_stats_mfma = resident_grid(compress_stats_mfma_kernel<B, U>);
  static const int cap_stats_valu = resident_grid(compress_stats_kernel<B, U>);
  static const int cap_quant_mfma = resident_grid(compress_quant_mfma_kernel<B, U>);
  static const int cap_quant_valu = resident_grid(compress_quant_kernel<B, U>);
  int cap = mfma ? cap_stats_mfma : cap_stats_valu;
  if (cap > kMaxPartials) cap = kMaxPartials;
  const int g = grid_for(nblocks, U, cap);
  hipLaunchKernelGGL(stats, dim3(g), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(x), nblocks, energy, alpha, partial);
  const int gq = grid_for(nblocks, U, mfma ? cap_quant_mfma : cap_quant_valu);
  if (mfma)
    hipLaunchKernelGGL((compress_quant_mfma_kernel<B, U>), dim3(gq), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(x), nblocks, energy, partial, g, scale,
                       reinterpret_cast<unsigned*>(q));
  else
    hipLaunchKernelGGL((compress_quant_kernel<B, U>), dim3(gq), dim3(kThreads), 0, stream,
                       static_cast<const uint4*>(x), nblocks, energy, partial, g, scale,
                       reinterpret_cast<uint2*>(q));
}

template <int B>
void launch_decompress(const uint8_t* q, const float* alpha, const float* scale, int64_t nblocks,
                       void* out, hipStream_t stream) {
  constexpr int U = unroll_decompress<B>();
  const int g = grid_for(nblocks, U, wg_cap());
  hipLaunchKernelGGL((decompress_kernel<B, U>), dim3(g), dim3(kThreads), 0, stream,
                     reinterpret_cast<const uint2*>(q), alpha, scale, nblocks,
                     static_cast<uint4*>(out));
}

template <int B>
void launch_decompress_sum(const Parts& parts, int nparts, int64_t nblocks, void* out,
                           hipStream_t stream) {
  constexpr int U = unroll_sum<B>();
  const int g = grid_for(nblocks, U, wg_cap());
  hipLaunchKernelGGL((decompress_sum_kernel<B, U>), dim3(g), dim3(kThreads), 0, stream,
                     parts, nparts, nblocks, static_cast<uint4*>(out));
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
    case TACO_ERR_BAD_ENGINE: return "TACO_ERR_BAD_ENGINE: unknown rotation engine";
  }
  return "TACO_ERR_UNKNOWN";
}

const char* taco_version(void) { return "0.2.0"; }

taco_status_t taco_set_rotation_engine(taco_engine_t engine) {
  if (engine != TACO_ENGINE_AUTO && engine != TACO_ENGINE_VALU && engine != TACO_ENGINE_MFMA)
    return TACO_ERR_BAD_ENGINE;
  g_engine = engine;
  return TACO_OK;
}

taco_engine_t taco_get_rotation_engine(void) { return static_cast<taco_engine_t>(g_engine); }

int64_t taco_num_scales(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK) return -1;
  return tokens * (hidden / block);
}

size_t taco_compress_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block) {
  if (check_shape(tokens, hidden, block) != TACO_OK) return 0;
  return static_cast<size_t>(kMaxPartials) * sizeof(float);
}

taco_status_t taco_compress(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                            float target_energy, uint8_t* q_fp8, float* alpha, float* scale,
                            void* workspace, size_t workspace_bytes, taco_stream_t stream) {
  if (!x_bf16 || !q_fp8 || !alpha || !scale || !workspace) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(x_bf16, 16) || !aligned(q_fp8, 16) || !aligned(alpha, 4) || !aligned(scale, 4) ||
      !aligned(workspace, 4))
    return TACO_ERR_ALIGN;
  if (!(target_energy >= 0x1p-40f && target_energy <= 0x1p40f)) return TACO_ERR_BAD_ENERGY;
  if (workspace_bytes < taco_compress_workspace_bytes(tokens, hidden, block)) return TACO_ERR_WORKSPACE;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  const int64_t nblocks = tokens * (hidden / block);
  float* partial = static_cast<float*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_compress<64>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, partial, s); break;
    case 128: launch_compress<128>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, partial, s); break;
    default: launch_compress<256>(x_bf16, nblocks, target_energy, q_fp8, alpha, scale, partial, s); break;
  }
  return launched();
}

taco_status_t taco_decompress(const uint8_t* q_fp8, const float* alpha, const float* scale,
                              int64_t tokens, int64_t hidden, int32_t block, void* y_bf16,
                              taco_stream_t stream) {
  if (!q_fp8 || !alpha || !scale || !y_bf16) return TACO_ERR_NULL;
  const taco_status_t st = check_shape(tokens, hidden, block);
  if (st != TACO_OK) return st;
  if (!aligned(q_fp8, 16) || !aligned(y_bf16, 16) || !aligned(alpha, 4) || !aligned(scale, 4))
    return TACO_ERR_ALIGN;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  const int64_t nblocks = tokens * (hidden / block);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_decompress<64>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
    case 128: launch_decompress<128>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
    default: launch_decompress<256>(q_fp8, alpha, scale, nblocks, y_bf16, s); break;
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
    parts.q[p] = reinterpret_cast<const uint2*>(q_fp8[p]);
    parts.alpha[p] = alpha[p];
    parts.scale[p] = scale[p];
  }
  if (!aligned(out_bf16, 16)) return TACO_ERR_ALIGN;
  if (device_cu_count() <= 0) return TACO_ERR_HIP;
  const int64_t nblocks = tokens * (hidden / block);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (block) {
    case 64: launch_decompress_sum<64>(parts, nparts, nblocks, out_bf16, s); break;
    case 128: launch_decompress_sum<128>(parts, nparts, nblocks, out_bf16, s); break;
    default: launch_decompress_sum<256>(parts, nparts, nblocks, out_bf16, s); break;
  }
  return launched();
}

}  // extern "C"
