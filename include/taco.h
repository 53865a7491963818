/*
 * libtaco -- TACO's fused FP8 compression operator for tensor-parallel
 * intermediate tensors, for AMD Instinct MI355X (gfx950).
 *
 * Sources.  "TACO pt-summary" is the Portuguese structured summary on
 * gist.science of "TACO: Efficient Communication Compression of Intermediate
 * Tensors for Scalable Tensor-Parallel LLM Training" (arXiv 2604.24088);
 * "TACO zh-news" is the Chinese euno.news summary of the same paper.
 *
 * Data model (every call):
 *   x      bf16 [tokens, hidden], row-major, contiguous.  N = tokens * hidden.
 *   block  B in {64, 128, 256}; hidden % B == 0.  Block k is the B consecutive
 *          elements [k*B, (k+1)*B) of the flattened tensor (always inside one row).
 *   q      uint8 [tokens, hidden]: OCP FP8 E4M3FN codes (bias 7, max 448).
 *   alpha  fp32 [tokens, hidden / B]: the per-block ASH scale.
 *   scale  fp32 [1]: the per-tensor DS scale s.
 * Compression computes, per block k,
 *   m_k     = (1/B) sum_i x_i^2                       (raw second moment)
 *   alpha_k = sqrt(E / m_k)      (1 if m_k == 0)      (ASH, to target energy E)
 *   y_k     = alpha_k * H_B x_k / sqrt(B)              (orthonormal Sylvester-Hadamard)
 * then s = 448 / max|y| over the whole tensor (1 if it is zero) and
 *   q = E4M3FN(s * y), round to nearest even, saturating at +-448.
 * Decompression returns bf16((1/alpha_k) * H_B (decode(q_k) / s) / sqrt(B)).
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer (HIP device memory of
 * the current device), including `scale`.  The caller owns every buffer; the
 * library allocates nothing.  x, q and the bf16 outputs must be 16-byte
 * aligned, the workspace 256-byte aligned, alpha and scale 4-byte aligned.
 *
 * Streams.  Every call only enqueues work on `stream` (NULL = the default
 * stream) and returns; outputs are valid once the stream reaches that point.
 * Calls that share a workspace must not run concurrently on different streams.
 *
 * Aliasing.  No output may overlap an input or another output (byte ranges
 * of the sizes below); inputs may overlap each other.  A violation returns
 * TACO_ERR_ALIAS.
 *
 * Errors.  Arguments are checked before anything is enqueued; a failed check
 * returns a nonzero status and enqueues nothing.  TACO_ERR_HIP reports a
 * failed kernel launch (hipGetLastError).  A device fault surfaces at the
 * caller's next synchronisation.  Inputs must be finite with |x| <= 2^56 and
 * every nonzero block must hold an element of magnitude >= 2^-56; E must lie in
 * [2^-40, 2^40].  Outside that domain results are unspecified (but no
 * out-of-bounds access happens).
 */
#ifndef TACO_H
#define TACO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t* taco_stream_t;

typedef enum {
  TACO_OK = 0,
  TACO_ERR_NULL = 1,              /* a required pointer is NULL                    */
  TACO_ERR_ALIGN = 2,             /* a pointer is not aligned as documented        */
  TACO_ERR_SHAPE = 3,             /* tokens < 1, hidden < 1 or hidden % block != 0 */
  TACO_ERR_UNSUPPORTED_BLOCK = 4, /* block not in {64, 128, 256}                   */
  TACO_ERR_BAD_ENERGY = 5,        /* target energy not finite or out of range      */
  TACO_ERR_WORKSPACE = 6,         /* workspace smaller than required               */
  TACO_ERR_BAD_NPARTS = 7,        /* nparts outside [1, TACO_MAX_PARTS]            */
  TACO_ERR_HIP = 8,               /* a HIP runtime call or kernel launch failed    */
  TACO_ERR_FLAGS = 9,             /* an unknown bit in a flags argument            */
  TACO_ERR_ALIAS = 10             /* an output overlaps an input or another output */
} taco_status_t;

/* Flags of taco_compress_ex and taco_decompress_sum_compress_ex. */
#define TACO_FLAG_TWO_PASS 1u
/* Default bound on the grid barrier's polls (barrier_polls == 0). */
#define TACO_DEFAULT_BARRIER_POLLS (1u << 16)

#define TACO_MAX_PARTS 8
/* amax buffers of taco_compress_delayed: TACO_AMAX_FLOATS fp32 (16 KiB) holding
 * TACO_AMAX_SLOTS slots, one per 256-byte line at index
 * i * (TACO_AMAX_FLOATS / TACO_AMAX_SLOTS); the other entries are never
 * written, so when zero-filled the max over the whole buffer is the max over
 * the slots. */
#define TACO_AMAX_SLOTS 64
#define TACO_AMAX_FLOATS 4096

/* Human-readable name of a status code (static storage, never NULL). */
const char* taco_status_string(taco_status_t status);

/* Library version string, e.g. "0.4.0" (0.4: per-call pass structure and
 * barrier bound; no process-wide settings). */
const char* taco_version(void);

/* Whether taco_compress of this shape runs as the single fused kernel on the
 * current device: 1 yes, 0 two kernels, -1 for an invalid shape or no usable
 * device.  The fused kernel holds the rotated
 * blocks in registers up to 16.8M elements, the bf16 input beyond that, up to
 * 25.2M elements at block 64 and 33.6M at blocks 128 and 256 on a 256-CU
 * MI355X; larger tensors take the two kernels. */
int taco_compress_is_single_pass(int64_t tokens, int64_t hidden, int32_t block);

/* Number of per-block ASH scales of a [tokens, hidden] tensor at this block
 * size (tokens * hidden / block), or -1 if the shape or block is invalid. */
int64_t taco_num_scales(int64_t tokens, int64_t hidden, int32_t block);

/* Bytes of device workspace taco_compress needs for this shape (0 for an
 * invalid shape; the same 37120 bytes for every valid one).  The workspace
 * holds the state of a grid-wide barrier (call counters and one slot per
 * workgroup) and per-workgroup partial maxima.
 * It must be zero-filled once when allocated; every call leaves it ready for
 * the next one.  Calls that share a workspace must be ordered (the same
 * stream).
 *
 * Residency.  The single-pass kernel (taco_compress, and taco_compress_ex
 * without TACO_FLAG_TWO_PASS) meets all its workgroups at a grid-wide barrier,
 * so they must all be resident at once: its grid is at most what the device
 * holds resident, and at most one workgroup per compute unit (the same for
 * the fused taco_decompress_sum_compress), and no other kernel may hold
 * compute units while it runs.  A
 * caller that overlaps compression with other kernels (e.g. a collective on
 * another stream) must pass TACO_FLAG_TWO_PASS, which never waits on another
 * workgroup.  If residency fails anyway, a workgroup gives up after
 * barrier_polls polls (TACO_DEFAULT_BARRIER_POLLS, tens of milliseconds, when
 * 0 is passed; a resident grid passes the barrier in microseconds), writes its
 * codes as E4M3 NaN (0x7F / 0xFF), so the failure cannot pass for a result,
 * and sets a sticky flag in the workspace (taco_workspace_timed_out).  The
 * fallback for the host: when the flag is set, clear it (zero the workspace)
 * and compress the same input again with TACO_FLAG_TWO_PASS; the two paths
 * give bitwise-identical results.  The workspace stays valid after a timeout. */
size_t taco_compress_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block);

/* Whether a single-pass call on this workspace (of taco_compress or
 * taco_decompress_sum_compress) has given up waiting at its grid barrier since
 * the workspace was zero-filled: *timed_out = 1 if so, else 0.  Waits for the
 * work queued on `stream` (NULL: the null stream) to finish, then reads 4
 * bytes of the workspace.  The flag is sticky: zero-fill the workspace to
 * clear it.  TACO_ERR_NULL for a NULL pointer, TACO_ERR_ALIGN for a workspace
 * not 256-byte aligned, TACO_ERR_HIP if the copy fails. */
taco_status_t taco_workspace_timed_out(const void* workspace, taco_stream_t stream, int* timed_out);

/*
 * Compress: energy -> ASH scale -> Hadamard rotation -> DS scale -> FP8
 * [TACO pt-summary, sections 2.B.1 (ASH), 2.B.2 (DS) and 2.B.3 (fused operator);
 *  the per-tensor DS scale follows TACO zh-news, method section].
 *   x_bf16          in : bf16 [tokens, hidden]
 *   target_energy   in : E, the energy every block is rescaled to (1.0 typical)
 *   q_fp8           out: uint8 [tokens, hidden]
 *   alpha           out: fp32 [tokens, hidden / block]
 *   scale           out: fp32 [1]
 *   workspace       scratch of at least taco_compress_workspace_bytes() bytes
 * One fused kernel when the tensor fits in the resident wavefronts (see
 * Residency above and taco_compress_is_single_pass), two kernels otherwise.
 * Same as taco_compress_ex with flags 0 and barrier_polls 0.
 */
taco_status_t taco_compress(const void* x_bf16, int64_t tokens, int64_t hidden,
                            int32_t block, float target_energy, uint8_t* q_fp8,
                            float* alpha, float* scale, void* workspace,
                            size_t workspace_bytes, taco_stream_t stream);

/*
 * taco_compress with the pass structure chosen by the caller, per call:
 *   flags          0, or TACO_FLAG_TWO_PASS: always the two kernels
 *                  (statistics, then quantisation re-reading x), which need
 *                  no co-residency; bitwise the same result.  Other bits:
 *                  TACO_ERR_FLAGS.
 *   barrier_polls  bound on the single-pass barrier's polls (0: the default,
 *                  TACO_DEFAULT_BARRIER_POLLS); a small bound makes waits give
 *                  up early (e.g. to exercise the timeout path in tests).
 */
taco_status_t taco_compress_ex(const void* x_bf16, int64_t tokens, int64_t hidden,
                               int32_t block, float target_energy, uint8_t* q_fp8,
                               float* alpha, float* scale, void* workspace,
                               size_t workspace_bytes, uint32_t flags,
                               uint32_t barrier_polls, taco_stream_t stream);

/*
 * taco_compress_ex without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is the library's own device
 * scratch, 37120 bytes per GPU (the size taco_compress_workspace_bytes gives
 * for every shape, so no shape is too large for it; a larger requirement would
 * return TACO_ERR_WORKSPACE), held until the process ends.  The call allocates
 * nothing; it looks the scratch up once per device, on the first call with that
 * device current.  Every call on a GPU shares that GPU's scratch: calls that
 * overlap on one GPU (on different streams) race, so they must be ordered.
 * Arguments, results, flags, barrier_polls and errors as taco_compress_ex;
 * a barrier timeout gives NaN codes as there, and its flag cannot be queried.
 */
taco_status_t taco_compress_noalloc(const void* x_bf16, int64_t tokens, int64_t hidden,
                                    int32_t block, float target_energy, uint8_t* q_fp8,
                                    float* alpha, float* scale, uint32_t flags,
                                    uint32_t barrier_polls, taco_stream_t stream);

/*
 * Decompress: decode -> undo s -> inverse rotation -> undo alpha -> bf16
 * [TACO pt-summary, section 2.B.2: both scales reverse the process].
 *   q_fp8, alpha, scale  in : the output of taco_compress (same shape / block)
 *   y_bf16               out: bf16 [tokens, hidden], round to nearest even
 */
taco_status_t taco_decompress(const uint8_t* q_fp8, const float* alpha,
                              const float* scale, int64_t tokens, int64_t hidden,
                              int32_t block, void* y_bf16, taco_stream_t stream);

/*
 * Decompress-and-sum: the local reduction of the two-shot (reduce-scatter +
 * all-gather) all-reduce [TACO pt-summary, section 2.B.3].
 *   out = bf16( sum_p decompress(q_p, alpha_p, scale_p) ), summed in fp32 and
 *   rounded once.
 *   q_fp8, alpha, scale  HOST arrays of `nparts` DEVICE pointers (read during
 *                        the call; the arrays may be freed when it returns)
 *   nparts               1 .. TACO_MAX_PARTS
 *   out_bf16             out: bf16 [tokens, hidden]; may not overlap any part
 *                        (TACO_ERR_ALIAS)
 */
taco_status_t taco_decompress_sum(const uint8_t* const* q_fp8, const float* const* alpha,
                                  const float* const* scale, int32_t nparts,
                                  int64_t tokens, int64_t hidden, int32_t block,
                                  void* out_bf16, taco_stream_t stream);

/* Bytes of device workspace taco_decompress_sum_compress needs: the compress
 * workspace (barrier state and partial maxima, zero-filled once, as for
 * taco_compress) followed by room for the bf16 sum, 2 * tokens * hidden bytes,
 * which the call uses when the reduced tensor does not fit on chip.  0 for an
 * invalid shape. */
size_t taco_decompress_sum_compress_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block);

/*
 * Decompress-sum-compress: the local step of the two-shot all-reduce with its
 * result compressed again for the all-gather leg [TACO pt-summary, section
 * 2.B.3: the compression kernels around the reduce-scatter and all-gather].
 *   Result = taco_compress(taco_decompress_sum(parts)): the bf16 sum of the
 *   parts' reconstructions (as taco_decompress_sum computes it) compressed
 *   with its own per-block alpha and per-tensor scale, bitwise equal to the
 *   two calls in sequence.  When the tensor fits on chip (and TACO_FLAG_TWO_PASS
 *   is not given to the _ex form) it is one kernel and the bf16 sum never
 *   reaches device memory; otherwise the sum goes through the workspace.
 *   q_fp8, alpha, scale   HOST arrays of `nparts` DEVICE pointers (1 ..
 *                         TACO_MAX_PARTS), as taco_decompress_sum
 *   target_energy         as taco_compress
 *   q_out, alpha_out, scale_out  out, as taco_compress; none may overlap an
 *                         input, another output or the workspace (TACO_ERR_ALIAS)
 *   workspace             at least taco_decompress_sum_compress_workspace_bytes(),
 *                         256-byte aligned, zero-filled once; same ordering and
 *                         residency rules as the taco_compress workspace
 */
taco_status_t taco_decompress_sum_compress(const uint8_t* const* q_fp8, const float* const* alpha,
                                           const float* const* scale, int32_t nparts,
                                           int64_t tokens, int64_t hidden, int32_t block,
                                           float target_energy, uint8_t* q_out,
                                           float* alpha_out, float* scale_out,
                                           void* workspace, size_t workspace_bytes,
                                           taco_stream_t stream);
/* The same with flags and barrier_polls as in taco_compress_ex. */
taco_status_t taco_decompress_sum_compress_ex(const uint8_t* const* q_fp8, const float* const* alpha,
                                              const float* const* scale, int32_t nparts,
                                              int64_t tokens, int64_t hidden, int32_t block,
                                              float target_energy, uint8_t* q_out,
                                              float* alpha_out, float* scale_out,
                                              void* workspace, size_t workspace_bytes,
                                              uint32_t flags, uint32_t barrier_polls,
                                              taco_stream_t stream);

/*
 * Single-pass Dual-Scale variants [TACO pt-summary, sections 2.B.2 (two scales
 * per block; the post-rotation scale keeps values inside the FP8 range) and
 * 2.B.3 (one fused kernel)].  Neither needs a tensor-wide maximum before
 * writing codes, so each is one streaming kernel with no workspace and no
 * residency requirement.
 *
 * Per-block overflow guard: alpha_k as in taco_compress; the post-rotation
 * scale is per block, s_k = 448 / max|y_k| when the block's rotated values
 * would exceed the FP8 range and 1 otherwise, so the target energy sets where
 * the values sit in the E4M3 range.
 *   scale_blk  out: fp32 [tokens, hidden / block], one s_k per block
 * taco_decompress_blockscale inverts it (scale_blk in place of the per-tensor
 * scale).
 */
taco_status_t taco_compress_blockscale(const void* x_bf16, int64_t tokens, int64_t hidden,
                                       int32_t block, float target_energy, uint8_t* q_fp8,
                                       float* alpha, float* scale_blk, taco_stream_t stream);
taco_status_t taco_decompress_blockscale(const uint8_t* q_fp8, const float* alpha,
                                         const float* scale_blk, int64_t tokens, int64_t hidden,
                                         int32_t block, void* y_bf16, taco_stream_t stream);

/*
 * Delayed per-tensor scale: s = 448 / amax_prev, where amax_prev is the
 * largest rotated value of an earlier tensor (1 if it is 0); rotated values
 * beyond the range saturate at +-448.  Decompress with taco_decompress.
 *   amax_prev  in : device, TACO_AMAX_FLOATS fp32; the earlier call's amax_out
 *                   (the max over its slots is used; all zeros means no history)
 *   scale      out: device fp32 [1], the s used
 *   amax_out   in/out: device, TACO_AMAX_FLOATS fp32; each slot becomes the
 *                   max of its content and part of this tensor's block maxima,
 *                   so zero-filled on entry it holds this tensor's largest |y|
 *                   as the max over the buffer.  May not overlap amax_prev
 *                   (TACO_ERR_ALIAS).
 */
taco_status_t taco_compress_delayed(const void* x_bf16, int64_t tokens, int64_t hidden,
                                    int32_t block, float target_energy, const float* amax_prev,
                                    uint8_t* q_fp8, float* alpha, float* scale, float* amax_out,
                                    taco_stream_t stream);

/*
 * INT8 degrade path: symmetric absmax INT8, the quantiser the pages compare
 * FP8 against [TACO pt-summary, sections 1 and 2.A: uniform INT8 steps map
 * the dense near-zero values of TP tensors to the same integer].  No ASH and
 * no rotation.  The pages give no INT8 arithmetic; this library uses
 *   A     = max |x| over the tensor (block == 0) or over each block of
 *           `block` consecutive elements of a row (block in {64, 128, 256})
 *   s     = fp32(127 / A), 1 if A == 0  (correctly rounded quotient)
 *   code  = clamp(round_half_even(x * s), -127, 127)
 *   x_hat = bf16_RNE(code / s)
 * where x * s and code / s are the exact product and quotient: each code and
 * each bf16 output is the correctly rounded value, decided without an fp32
 * intermediate rounding.
 *
 *   x_bf16     in : bf16 [tokens, hidden], 16-byte aligned; hidden % 8 == 0
 *                   when block == 0, hidden % block == 0 otherwise
 *   q_int8     out: int8 [tokens, hidden], 16-byte aligned
 *   scale      out: fp32 [1] (block == 0) or [tokens, hidden / block]
 *   workspace  block == 0: device scratch of at least
 *              taco_compress_int8_workspace_bytes() bytes, 256-byte aligned
 *              (it holds per-workgroup maxima; no zero-fill needed; a
 *              taco_compress workspace may be passed, its barrier state is
 *              not touched).  Ignored (may be NULL) for block != 0.
 * Errors: TACO_ERR_NULL, TACO_ERR_SHAPE, TACO_ERR_UNSUPPORTED_BLOCK (block
 * not in {0, 64, 128, 256}), TACO_ERR_ALIGN, TACO_ERR_WORKSPACE,
 * TACO_ERR_HIP.  Per-tensor calls are two kernels (maxima, then codes), so
 * x is read twice; per-block calls are one.
 */
size_t taco_compress_int8_workspace_bytes(int64_t tokens, int64_t hidden, int32_t block);
taco_status_t taco_compress_int8(const void* x_bf16, int64_t tokens, int64_t hidden, int32_t block,
                                 int8_t* q_int8, float* scale, void* workspace,
                                 size_t workspace_bytes, taco_stream_t stream);

/* INT8 decompress: y_bf16 (bf16 [tokens, hidden], 16-byte aligned) from the
 * codes and the scale(s) of taco_compress_int8 with the same block (0: one
 * scale per tensor).  Same errors, no workspace. */
taco_status_t taco_decompress_int8(const int8_t* q_int8, const float* scale, int64_t tokens,
                                   int64_t hidden, int32_t block, void* y_bf16,
                                   taco_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TACO_H */
