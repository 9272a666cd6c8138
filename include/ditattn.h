/*
 * ditattn.h -- C ABI of the DiT attention library for AMD Instinct MI355X (gfx950).
 *
 * Three operations, all non-causal and all on one GPU (and, further below, the extended
 * attention calls and the First Block Cache step built around resid_rel_l1):
 *
 *   attn_fwd_bf16    O = softmax(Q K^T * scale) V per (batch, head), QK^T and PV on bf16
 *                    matrix cores.  The DiT self-attention that the "Diffusion Attention
 *                    Backends" page (vLLM-Omni, Overview and Backend Options) dispatches to
 *                    FlashAttention / scaled_dot_product_attention, computed blockwise
 *                    on chip as the "Flash Attention 2 for Z-Image S3-DiT" page (hotdry blog,
 *                    method paragraph) describes; the flash-attention op is 73.76% of a video
 *                    DiT's FLOPs in the FLOP table of the "TMAP image-to-video inference
 *                    acceleration" page (section on overlapping communication).
 *   attn_fwd_int8qk  The same attention with Q and K quantized to int8 (8-bit attention as in
 *                    the TMAP page's SageAttention section and the SAGE_ATTN backend), with the
 *                    zero-scale guard of the TMAP page's operator-details section; PV stays
 *                    bf16.
 *   resid_rel_l1     sum|a - b| / sum|b| over two residual tensors: the first-block residual
 *                    difference that First Block Cache compares with its threshold
 *                    ("ParaAttention" page, First Block Cache section).
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers, allocated and owned by the caller.  The library
 *     allocates no memory and keeps no state between calls.
 *   - Every tensor is 16-byte aligned and, except in the *_ex calls (strided views), contiguous
 *     and row-major.
 *   - Attention tensors are [B, H, S, D]: batch, head, token, channel (channel fastest).
 *     Q, K, V are bf16 (raw 16-bit patterns); O is fp32 (the *_ex calls: fp32 or bf16).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Each call only enqueues work on
 *     it and returns; results are valid once the caller synchronises with the stream.
 *   - Return value: DITATTN_OK (0) or a negative status.  Arguments are validated before any
 *     work is enqueued, so on DITATTN_EINVAL / EUNSUPPORTED / EWORKSPACE nothing was launched
 *     and no HIP call was made.  DITATTN_EHIP means the HIP runtime rejected a launch.
 *   - Inputs are assumed finite; NaN or Inf inputs give unspecified outputs.
 *   - Calls are thread-safe and re-entrant; concurrent calls that share a workspace or an
 *     output buffer race.
 */
#ifndef DITATTN_H
#define DITATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DITATTN_API __attribute__((visibility("default")))
#else
#define DITATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum ditattn_status {
  DITATTN_OK = 0,
  DITATTN_EINVAL = -1,       /* null or misaligned pointer, size < 1, scale not finite > 0 */
  DITATTN_EUNSUPPORTED = -2, /* head dim D other than 64 or 128 */
  DITATTN_EWORKSPACE = -3,   /* workspace NULL or smaller than the *_workspace_bytes value */
  DITATTN_EHIP = -4          /* the HIP runtime reported an error for a launch */
};

/* Exact attention, bf16 in / fp32 out.
 *   q, k, v : bf16 [B, H, S, D] device pointers (read only)
 *   o       : fp32 [B, H, S, D] device pointer (written; must not alias q, k, v)
 *   B, H, S : >= 1;  D : 64 or 128
 *   scale   : finite and > 0; callers pass 1/sqrt(D), the scaled_dot_product_attention default
 * o[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:] . k[b,h,j,:]) * v[b,h,j,:], all j < S.
 * Accumulation is fp32; the softmax weights are rounded to bf16 for the PV product. */
DITATTN_API int attn_fwd_bf16(const void* q, const void* k, const void* v, float* o,
                  int B, int H, int S, int D, float scale, void* stream);

/* Workspace of attn_fwd_int8qk, in bytes, for the given shape (0 if the shape is invalid).
 * Layout, each segment starting on a 256-byte boundary, in this order:
 *   [0] k_mean  fp32 [B, H, D]            per-channel mean of K over the S tokens
 *   [1] q_scale fp32 [B, H, ceil(S/128)]  one scale per 128-token block of Q
 *   [2] k_scale fp32 [B, H, ceil(S/64)]   one scale per 64-token block of smoothed K
 *   [3] q_codes int8 [B, H, S, D]
 *   [4] k_codes int8 [B, H, S, D]
 *   [5] scratch  fp64 pairs used while forming k_mean, then the attention's tail workspace
 *                and, at D = 128 and S >= 32768, the V^T tiles of V (see attn_fwd_bf16_ws;
 *                contents unspecified)
 * After a successful call segments [0]-[4] hold the values the attention used. */
DITATTN_API size_t attn_int8qk_workspace_bytes(int B, int H, int S, int D);

/* Byte offsets of the six workspace segments above; returns the total size like
 * attn_int8qk_workspace_bytes (0 and offsets untouched if the shape is invalid). */
DITATTN_API size_t attn_int8qk_workspace_offsets(int B, int H, int S, int D, size_t offsets[6]);

/* Attention with int8 Q and K and bf16 PV.
 *   q, k, v, o, B, H, S, D, scale : as attn_fwd_bf16
 *   workspace       : device buffer of >= attn_int8qk_workspace_bytes(B, H, S, D) bytes,
 *                     256-byte aligned, owned by the caller (layout above)
 * Steps, in stream order:
 *   1. k_mean[b,h,d] = fp32( fp64(exact sum over s of K[b,h,s,d]) / S ).  The sum is carried
 *      as an exact double-double, so the result is the correctly rounded fp64 sum, divided in
 *      fp64 and rounded once to fp32 (exact whenever a channel's values span < 2^100).
 *   2. Ks = fp32(K) - k_mean (one fp32 subtraction).  Q is not smoothed.
 *   3. Per block (Q: 128 tokens, K: 64 tokens, within one (b, h); a tail block holds only the
 *      valid tokens): amax = max|x|, scale = amax / 127 (IEEE fp32 division); amax == 0 gives
 *      scale = 1.0 so an all-zero block never divides by zero.
 *      code = clamp(round_half_even(x / scale), -127, 127), x / scale an IEEE fp32 division.
 *   4. s_ij = (integer dot of the codes) * q_scale * k_scale * scale, online softmax, and
 *      PV on bf16 matrix cores with fp32 accumulation, o in fp32. */
DITATTN_API int attn_fwd_int8qk(const void* q, const void* k, const void* v, float* o,
                    int B, int H, int S, int D, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Attention with fp8 (OCP e4m3) Q and K and bf16 PV: the int8 call's steps with e4m3 codes.
 * The pages run their linear layers in fp8 and their attention in 8 bits; CDNA4's fp8 matrix
 * cores (v_mfma_f32_32x32x64_f8f6f4) run at the int8 rate, and a floating-point grid keeps
 * small values of a block that holds an outlier.
 *   arguments as attn_fwd_int8qk; the workspace has the same size and layout
 *   (attn_int8qk_workspace_bytes / _offsets), its code segments holding e4m3 bytes
 * Steps 1-2 as attn_fwd_int8qk; then per block amax = max|x|, scale = amax / 448 (IEEE fp32
 * division; 448 is the largest finite e4m3 value), 1.0 if amax == 0;
 * code = e4m3(clamp(x / scale, -448, 448)), x / scale an IEEE fp32 division, one rounding to
 * e4m3 (nearest, ties to even; e4m3 has 3 fraction bits, exponent bias 7, subnormals below
 * 2^-6).  s_ij = (sum_d qc_id kc_jd, products exact, fp32 accumulation) * q_scale * k_scale *
 * scale; softmax and PV as attn_fwd_int8qk. */
DITATTN_API int attn_fwd_fp8qk(const void* q, const void* k, const void* v, float* o,
                   int B, int H, int S, int D, float scale,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Attention with fp8 for both products (D = 128): Q and K as attn_fwd_fp8qk, and V as e4m3
 * codes with one scale per (b, h, channel) over all S tokens, so PV runs on the fp8 matrix
 * cores as well (about half the matrix-core time of the bf16 call).
 *   arguments as attn_fwd_int8qk; D must be 128 (else DITATTN_EUNSUPPORTED)
 *   workspace : >= attn_fp8_workspace_bytes(B, H, S, D) bytes, 256-byte aligned; segments
 *               [0]-[5] as the int8 call's (codes e4m3), then
 *               [6] v_scale fp32 [B, H, D]   amax over the tokens / 448 (1.0 for amax == 0)
 *               [7] v_codes e4m3 [B, H, S, D]  e4m3(clamp(V / v_scale, -448, 448)), one rounding
 *               [8] scratch (partial channel maxima)
 * o[b,h,i,d] = sum_j p_ij vq[b,h,j,d] v_scale[b,h,d] / sum_j p_ij with p the softmax weights of
 * the fp8 scores.  Each weight enters the product rounded to e4m3 at the kernel's running
 * offset (at most 2^-4 relative), and the row sum adds those same rounded weights, so the
 * weights of a row sum to one (a V constant over the keys comes back unchanged). */
DITATTN_API size_t attn_fp8_workspace_bytes(int B, int H, int S, int D);
DITATTN_API size_t attn_fp8_workspace_offsets(int B, int H, int S, int D, size_t offsets[9]);
DITATTN_API int attn_fwd_fp8(const void* q, const void* k, const void* v, float* o,
                 int B, int H, int S, int D, float scale,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ---- extended attention calls: strided views, bf16 output, per-row log-sum-exp --------------
 *
 * Same operations as attn_fwd_bf16 / attn_fwd_int8qk, with three additions that the steps
 * around the kernel need:
 *   strides   : 12 int64 element strides, for q, k, v, o in this order, each as (batch, head,
 *               token); the channel axis must be contiguous.  A contiguous [B, H, S, D] tensor
 *               is {H*S*D, S*D, D}; a [B, S, H, D] tensor (heads interleaved per token) is
 *               {S*H*D, D, H*D}.  Every stride >= 0 and a multiple of 16 bytes' worth of
 *               elements (8 for bf16, 4 for fp32); token strides of q, k, v below 2^24.
 *   out_dtype : DITATTN_OUT_F32 (o fp32) or DITATTN_OUT_BF16 (o bf16, each value the fp32
 *               result rounded to nearest even)
 *   lse       : NULL, or fp32 [B, H, S] contiguous, 4-byte aligned, receiving
 *               lse[b,h,i] = log sum_j exp(s_ij) with s_ij the scaled score of that call (the
 *               int8 call: of the quantized scores).  Partial results over disjoint key sets
 *               merge through it: lse = log(e^lse_A + e^lse_B), o = e^(lse_A-lse) o_A +
 *               e^(lse_B-lse) o_B — how a sequence split over devices (the ring dimension of
 *               the context-parallel mesh, "ParaAttention" page, Context Parallelism section)
 *               combines partial outputs.
 * o and lse must not overlap q, k, v or each other, and o's strides must not map two rows to
 * one address (identical pointers are rejected; other overlaps are the caller's to avoid).
 * Errors as the plain calls, plus
 * DITATTN_EINVAL for a NULL strides array, a bad out_dtype, or a stride that breaks the
 * rules above. */
#define DITATTN_OUT_F32 0
#define DITATTN_OUT_BF16 1

DITATTN_API int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o,
                                 int out_dtype, float* lse, const int64_t* strides,
                                 int B, int H, int S, int D, float scale, void* stream);

/* As attn_fwd_bf16_ex, with a workspace that lets the call share its last round of query
 * tiles out over every CU.  The calls above run one workgroup (one CU) per tile of 256 query
 * rows of one (b, h); when the B * H * ceil(S / 256) tiles are not a multiple of the CU count
 * the last round leaves CUs idle (1024^2 images, B1 H24 S4608: 432 tiles on 256 CUs).  Here
 * the tiles of that last round are cut along the key axis into equal ranges, one per CU, and
 * the partial results of a tile are merged exactly as the extended calls describe (running
 * maximum and sum: the online softmax of the "Flash Attention 2 for Z-Image S3-DiT" page,
 * method paragraph, applied across parts), in a fixed order, so the output does not depend on
 * timing.  Tiles of the full rounds are computed exactly as attn_fwd_bf16 computes them; in
 * the last round each tile's sums over the keys are formed in parts and then merged.  At D =
 * 128 and S >= 32768 the workspace also holds a transposed copy of V in 64-key tiles, written
 * by the call, from which the PV products read their operand with one LDS read instead of
 * two; the products are the same (same values, same order), so this changes no output bit.
 *   workspace : device buffer of >= attn_bf16_workspace_bytes(B, H, S, D) bytes, 256-byte
 *               aligned, caller owned, contents unspecified before and after; calls that use
 *               one workspace at the same time (on different streams) race
 * Errors as attn_fwd_bf16_ex, plus DITATTN_EWORKSPACE. */
DITATTN_API size_t attn_bf16_workspace_bytes(int B, int H, int S, int D);
DITATTN_API int attn_fwd_bf16_ws(const void* q, const void* k, const void* v, void* o,
                                 int out_dtype, float* lse, const int64_t* strides,
                                 int B, int H, int S, int D, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* As attn_fwd_int8qk with the additions above; the workspace (size and layout) is the same,
 * its codes stay contiguous [B, H, S, D] whatever the strides of q and k. */
DITATTN_API int attn_fwd_int8qk_ex(const void* q, const void* k, const void* v, void* o,
                                   int out_dtype, float* lse, const int64_t* strides,
                                   int B, int H, int S, int D, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* As attn_fwd_fp8qk with the additions above (lse of the fp8 scores). */
DITATTN_API int attn_fwd_fp8qk_ex(const void* q, const void* k, const void* v, void* o,
                                  int out_dtype, float* lse, const int64_t* strides,
                                  int B, int H, int S, int D, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* As attn_fwd_fp8 with the additions above. */
DITATTN_API int attn_fwd_fp8_ex(const void* q, const void* k, const void* v, void* o,
                                int out_dtype, float* lse, const int64_t* strides,
                                int B, int H, int S, int D, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of resid_rel_l1, in bytes, for n elements (0 if n < 1). */
DITATTN_API size_t resid_rel_l1_workspace_bytes(int64_t n);

/* Relative L1 distance of two residuals.
 *   a, b      : bf16 device arrays of n elements each (any shape, flattened), 16-byte aligned
 *   n         : >= 1
 *   out       : fp32 device scalar, written with sum|a - b| / sum|b| (b is the reference);
 *               if sum|b| == 0 it is 0 when the numerator is 0, else +inf
 *   workspace : device buffer of >= resid_rel_l1_workspace_bytes(n) bytes, caller owned
 * Per-thread partial sums are fp32, combined in fp64 in a fixed order, so the result is
 * deterministic for a given n. */
DITATTN_API int resid_rel_l1(const void* a, const void* b, int64_t n, float* out,
                 void* workspace, size_t workspace_bytes, void* stream);

/* resid_rel_l1 for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments without the workspace,
 * same kernels, same result bits.  The partial sums go to a 64 KiB array in the library's own
 * device memory instead: one copy per GPU, held from the library's load until the process ends.
 * Every n fits (the pass uses at most 4096 partial pairs); a need beyond the array would be
 * rejected with DITATTN_EWORKSPACE.  The call makes no allocation; its first call on a GPU
 * looks up that GPU's copy of the array (hipGetSymbolAddress; DITATTN_EHIP if that fails).
 * All calls on one GPU share the array: calls that overlap on a GPU (on different streams, or
 * from threads without stream ordering) race and give wrong results.  `stream` may belong to
 * any device; the array of that stream's device is used. */
DITATTN_API int resid_rel_l1_noalloc(const void* a, const void* b, int64_t n, float* out,
                                     void* stream);

/* ---- quantization-error probe -----------------------------------------------------------
 *
 * Which attention layers may run quantized: the "TMAP image-to-video inference acceleration"
 * page (section on preserving video quality) keeps the layers whose quantized attention
 * errs most in full precision.  attn_quant_probe measures that error for one call: the bf16
 * path's output on n_rows evenly spaced query rows per (b, h) against the output o_q of a
 * quantized call (attn_fwd_int8qk[_ex]) on the same inputs, at about n_rows / S of a bf16
 * call's work.  Sampled row i = step / 2 + i * step with step = floor(S / n_rows): the middle
 * row of the i-th bin of step rows (integer division). */

/* Number of uniform key chunks ns the probe splits each (b, h) into (0 if the arguments are
 * invalid): enough to give the few sampled rows work for every CU.  Chunk c < ns holds keys
 * [c L, (c + 1) L) with L = 64 floor(floor(S / ns) / 64) (L = S when ns = 1); chunk ns holds
 * the remaining keys [ns L, S), if any. */
DITATTN_API int attn_quant_probe_splits(int B, int H, int S, int D, int n_rows);

/* Workspace of attn_quant_probe, in bytes (0 if the shape or n_rows is invalid).  Layout, each
 * segment on a 256-byte boundary: fp32 [B][ns + 1][H][n_rows][D] chunk outputs, fp32
 * [B][ns + 1][H][n_rows] chunk log-sum-exps, fp64 [B*H][ceil(n_rows / 8)][2] partial sums.  After a call the
 * chunk segments hold the bf16 path's partial results for the sampled rows (chunk ns only if
 * it has keys). */
DITATTN_API size_t attn_quant_probe_workspace_bytes(int B, int H, int S, int D, int n_rows);

/*   q, k, v, strides, B, H, S, D, scale : the quantized call's inputs, as in attn_fwd_bf16_ex
 *   o_q, o_q_dtype                      : its output (DITATTN_OUT_F32 / _BF16), strides[9..11]
 *   n_rows                              : 1 <= n_rows <= S
 *   err       : fp32 device array of 1 + B*H values, written with
 *               err[0]          = sqrt(sum |o_q - o|^2 / sum |o|^2) over all sampled rows,
 *               err[1 + b*H + h] the same for head (b, h), o = the bf16 path's output
 *   workspace : >= attn_quant_probe_workspace_bytes(B, H, S, D, n_rows) bytes, 256-byte aligned
 * Errors as attn_fwd_bf16_ex, plus DITATTN_EINVAL for n_rows out of range, a NULL err, or
 * q's token stride times step reaching 2^24 (the sampled rows are read as a strided view). */
DITATTN_API int attn_quant_probe(const void* q, const void* k, const void* v, const void* o_q,
                                 int o_q_dtype, const int64_t* strides, int B, int H, int S,
                                 int D, float scale, int n_rows, float* err, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---- First Block Cache ------------------------------------------------------------------
 *
 * A denoising step of a DiT may skip its remaining transformer blocks when the residual its
 * first block adds differs little from the one it added at the latest computed step; it then
 * reuses the residual the remaining blocks added at that step ("ParaAttention" page, First
 * Block Cache section; parameters as the DBCache parameters of the "Cache-DiT acceleration"
 * page, vLLM-Omni user guide).  Per step, on the caller's stream:
 *   r1 = resid_sub(h1, h0)                       h0: step input, h1: first block's output
 *   fbcache_decide(r1, r1_ref, ...)              r1_ref: r1 of the latest computed step
 *   use_cache (state, device) == 1:  out = resid_add(h1, rest)           -- skip the blocks
 *                           == 0:  hN = remaining blocks(h1); rest = resid_sub(hN, h1);
 *                                  r1_ref = r1 (swap two residual buffers, no copy)
 * The caller reads the 4-byte decision from device memory to branch (one synchronisation). */

/* Cache policy (host memory, read at each call). */
typedef struct ditattn_fbcache_config {
  float residual_diff_threshold;       /* reuse only when the difference is below this (fp32) */
  int32_t max_warmup_steps;            /* steps 0 .. max_warmup_steps-1 always compute (>= 0) */
  int32_t max_cached_steps;            /* at most this many cached steps in the run; -1: no cap */
  int32_t max_continuous_cached_steps; /* at most this many cached steps in a row; -1: no cap */
} ditattn_fbcache_config;

/* Per-run state, in DEVICE memory (32 bytes, 4-byte aligned, caller owned).  All zero before
 * the first step of a run; each fbcache_decide call advances it by one step. */
typedef struct ditattn_fbcache_state {
  int32_t steps;                    /* steps decided so far */
  int32_t cached_steps;             /* of them, served from the cache */
  int32_t continuous_cached_steps;  /* cached steps since the latest computed step */
  int32_t use_cache;                /* decision of the latest step: 1 reuse, 0 compute */
  float diff;                       /* that step's difference (NaN: no reference residual) */
  int32_t reserved[3];
} ditattn_fbcache_state;

/* One step's cache decision.
 *   resid       : bf16 device array of n elements, this step's first-block residual
 *   prev_resid  : the reference residual (bf16, n elements), or NULL when there is none yet
 *                 (the step then computes)
 *   n           : >= 1
 *   cfg         : host pointer; threshold finite and >= 0, warmup >= 0, caps >= -1
 *   state       : device pointer to the run's ditattn_fbcache_state
 *   workspace   : device buffer of >= resid_rel_l1_workspace_bytes(n) bytes (may be NULL when
 *                 prev_resid is NULL)
 * The difference is resid_rel_l1(resid, prev_resid) (same kernel, same value).  The step
 * reuses the cache iff steps >= max_warmup_steps, a reference exists, diff < threshold (false
 * for NaN), cached_steps < max_cached_steps (or no cap) and continuous_cached_steps <
 * max_continuous_cached_steps (or no cap).  Calls on one state must be ordered (one stream). */
DITATTN_API int fbcache_decide(const void* resid, const void* prev_resid, int64_t n,
                               const ditattn_fbcache_config* cfg, ditattn_fbcache_state* state,
                               void* workspace, size_t workspace_bytes, void* stream);

/* out = a + b and out = a - b over n bf16 values (device arrays, 16-byte aligned, n >= 1),
 * each result the exact value rounded once to bf16 (nearest, ties to even).  out may be a or b
 * itself; any other overlap is rejected (DITATTN_EINVAL). */
DITATTN_API int resid_add(const void* a, const void* b, void* out, int64_t n, void* stream);
DITATTN_API int resid_sub(const void* a, const void* b, void* out, int64_t n, void* stream);

/* Static English description of a status code (never NULL). */
DITATTN_API const char* ditattn_status_string(int status);

/* ---- calibration (measurement support, not part of the attention path) ------------------
 *
 * For the callers that report attention throughput against the matrix cores' capability (the
 * benchmark): the nominal dense peaks assume the rated clock, which a power-limited chip does
 * not hold under dense products on real data.  ditattn_mfma_probe launches 1024 workgroups of
 * 512 threads (8 wavefronts, two per SIMD on every CU of a 256-CU part, four rounds); every
 * wavefront issues iters x 8 independent 32x32 matrix products back to back and nothing else:
 *   dtype 0: v_mfma_f32_32x32x16_bf16 (32768 flops each); 1: v_mfma_i32_32x32x32_i8 (65536 ops)
 *   random_operands 1: per-lane random operand values; 0: constant ones
 *   iters  : >= 1
 *   clocks : int64 device buffer of >= 2048 entries, caller owned: clocks[2 w] = shader clocks
 *            workgroup w ran for, clocks[2 w + 1] = 100 MHz reference clocks over the same
 *            interval (their ratio x 100 MHz is the shader clock it ran at)
 * The caller times the launch on `stream`; the work is 1024 x 8 x iters x 8 products.
 * DITATTN_EINVAL for other dtype / random_operands values, iters < 1 or a null or misaligned
 * clocks pointer. */
DITATTN_API int ditattn_mfma_probe(int dtype, int random_operands, int iters, int64_t* clocks,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DITATTN_H */
