// Host-side launchers of the gfx950 kernels (internal to the library; the public C ABI is
// include/ditattn.h).  Each launcher only enqueues work on `stream` and returns the HIP error
// of the launch.  Shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ditattn.h"

namespace ditattn {

// Element strides of a [B, H, S, D] tensor view: batch, head, token.  The channel axis is
// contiguous.
struct Strides {
  int64_t b, h, s;
};

// One attention call: q, k, v bf16 views, o fp32 or bf16 view, optional lse fp32 [B, H, Sq].
// S keys and Sq query rows per (b, h) (Sq = S except for the quantization probe's sampled
// rows; the int8 path always has Sq = S).
struct AttnCall {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  bool o_bf16;
  float* lse;
  Strides qs, ks, vs, os;
  int B, H, S, D;
  float scale;
  int Sq;
  // attn_tail_bytes(S, D) bytes of device memory (256-byte aligned) in which the launch shares
  // its last, partly filled round of query tiles out over every CU; null: whole tiles only.
  void* tail;
  // attn_vt_bytes(B, H, S, D) bytes (256-byte aligned, apart from `tail`) for the V^T tiles a
  // long launch with bf16 V reads V through; null: V read as it is.
  void* vt;
};

// Bytes of the tail workspace of an attention launch over S keys (0 when no launch over S keys
// can have a tail phase).
size_t attn_tail_bytes(int S, int D);

// Bytes of the V^T tiles of a launch with bf16 V over [B, H, S, D] (0 when it reads V as it is:
// D = 64, or S below the length from which the tiles pay).
size_t attn_vt_bytes(int B, int H, int S, int D);

hipError_t launch_attn_bf16(const AttnCall& ac, hipStream_t stream);

// The int8-QK attention on the prepass's contiguous codes and scales (V, O, lse from `ac`).
hipError_t launch_attn_int8(const AttnCall& ac, const int8_t* q_codes, const int8_t* k_codes,
                            const float* q_scale, const float* k_scale, hipStream_t stream);

// The fp8-QK attention: as launch_attn_int8 with e4m3 codes (QK on the fp8 matrix cores).
hipError_t launch_attn_fp8(const AttnCall& ac, const uint8_t* q_codes, const uint8_t* k_codes,
                           const float* q_scale, const float* k_scale, hipStream_t stream);

// fp8 for both products (D = 128 only): e4m3 Q/K codes as launch_attn_fp8, V as e4m3 codes
// (contiguous [B, H, S, D]) with one scale per (b, h, channel); PV on the fp8 matrix cores.
hipError_t launch_attn_fp8_all(const AttnCall& ac, const uint8_t* q_codes, const uint8_t* k_codes,
                               const uint8_t* v_codes, const float* q_scale, const float* k_scale,
                               const float* v_scale, hipStream_t stream);

// Number of token chunks the K-mean partial pass splits each (b, h) into.
int kmean_chunks(int B, int H, int S);

// The int8 prepass: K channel mean (exact double-double sum, one division, one rounding to
// fp32) and per-block int8 quantization of Q (128-token blocks) and of the mean-smoothed K
// (64-token blocks).  Three launches: mean partial sums together with the Q blocks, the mean,
// then the K blocks.  partial: scratch of B*H*kmean_chunks(B,H,S)*D double pairs.  fp8: the
// codes are fp8 e4m3 (scale = amax / 448, one rounding to e4m3) instead of int8.
hipError_t launch_prepass(const void* q, Strides qs, const void* k, Strides ks, float* k_mean,
                          double* partial, int8_t* q_codes, int8_t* k_codes, float* q_scale,
                          float* k_scale, int B, int H, int S, int D, bool fp8, hipStream_t stream);

// fp8 V (D = 128): per-(b, h, channel) amax of |V| over the S tokens (partials of
// kmean_chunks token chunks: B*H*chunks*D floats in `partial`), v_scale = amax / 448 (1.0 for a
// zero channel), and e4m3 codes of V / v_scale into the contiguous [B, H, S, D] v_codes.
hipError_t launch_vquant(const void* v, Strides vs, float* v_scale, float* partial,
                         uint8_t* v_codes, int B, int H, int S, int D, hipStream_t stream);

// Number of partial-sum workgroups the relative-L1 pass uses for n elements.
int rel_l1_blocks(int64_t n);

hipError_t launch_rel_l1(const void* a, const void* b, int64_t n, float* out, double* partial,
                         hipStream_t stream);

// Partial pairs the static scratch array of launch_rel_l1_static holds.
size_t rel_l1_static_pairs();

// launch_rel_l1 with the partial pairs in the library's static per-device array (no
// allocation, no workspace); calls that overlap on one GPU race.
hipError_t launch_rel_l1_static(const void* a, const void* b, int64_t n, float* out,
                                hipStream_t stream);

// The relative-L1 pass of resid against prev_resid (skipped when prev_resid is null) followed by
// one First Block Cache decision on *state (device memory).  partial: rel_l1_blocks(n) pairs.
hipError_t launch_fbcache_decide(const void* resid, const void* prev_resid, int64_t n,
                                 const ditattn_fbcache_config& cfg, ditattn_fbcache_state* state,
                                 double* partial, hipStream_t stream);

// Key chunks the quantization probe splits each (b, h) into for R sampled rows.
int probe_splits(int B, int H, int S, int R);

// The probe's chunks: ns chunks of L keys (L a multiple of 64, or L = S when ns = 1), then
// `tail` = S - ns L remaining keys as chunk ns (none when tail = 0).
struct ProbeChunks {
  int ns, L, tail;
};
ProbeChunks probe_chunks(int B, int H, int S, int R);

// Row groups of the probe's merge (its sums workspace holds B*H*groups double pairs).
int probe_row_groups(int R);

// The quantization probe: bf16 attention of R rows per (b, h), rows step/2 + i step with
// step = S / R (q, k, v, scale and their strides from `base`), over the probe_chunks chunks of
// keys, each with its lse: part fp32 [B][ns + 1][H][R][D], lse fp32 [B][ns + 1][H][R]; then
// err[1 + bh] (and err[0] over all) = sqrt(sum |o_q - o|^2 / sum |o|^2) against the quantized
// output o_q on those rows.  sums: B*H*probe_row_groups(R) double pairs.
hipError_t launch_quant_probe(const AttnCall& base, const void* o_q, bool o_q_bf16, Strides oqs,
                              int R, float* err, float* part, float* lse, double* sums,
                              hipStream_t stream);

// Calibration (not part of the attention path): mfma_probe_workgroups() workgroups of 8
// wavefronts, each issuing iters x 8 independent 32x32 products (bf16 or int8) on random or
// constant operands; clocks[2 w], clocks[2 w + 1]: shader and 100 MHz reference clocks of
// workgroup w.
int mfma_probe_workgroups();
hipError_t launch_mfma_probe(bool int8, bool random, int iters, int64_t* clocks, hipStream_t stream);

// out = bf16(a + b) (SUB: a - b) elementwise over n bf16 values, each rounded once.
hipError_t launch_resid_addsub(const void* a, const void* b, void* out, int64_t n, bool sub,
                               hipStream_t stream);

}  // namespace ditattn
