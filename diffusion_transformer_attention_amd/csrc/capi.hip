// C ABI of the library (declared in include/ditattn.h): argument validation, workspace
// layout and kernel launches on the caller's stream.  Validation never touches the HIP
// runtime, so a rejected call enqueues nothing and needs no GPU.
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "ditattn.h"
#include "kernels.h"

namespace {

constexpr size_t kSegAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape checks shared by the attention entry points.  Grid sizes must fit the 32-bit grid.
int check_attn_shape(int B, int H, int S, int D) {
  if (B < 1 || H < 1 || S < 1) return DITATTN_EINVAL;
  if (D != 64 && D != 128) return DITATTN_EUNSUPPORTED;
  const long long bh = (long long)B * H;
  const long long tiles = bh * ((S + 127LL) / 128 + (S + 63LL) / 64);
  if (tiles > 0x7FFFFFFFLL) return DITATTN_EINVAL;
  return DITATTN_OK;
}

int check_attn_args(const void* q, const void* k, const void* v, const float* o, int B, int H,
                    int S, int D, float scale) {
  if (!q || !k || !v || !o) return DITATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DITATTN_EINVAL;
  if (static_cast<const void*>(o) == q || static_cast<const void*>(o) == k ||
      static_cast<const void*>(o) == v)
    return DITATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return DITATTN_EINVAL;
  return check_attn_shape(B, H, S, D);
}

int status_of(hipError_t e) { return e == hipSuccess ? DITATTN_OK : DITATTN_EHIP; }

// Strides of the extended calls: non-negative, 16-byte multiples, token strides of the inputs
// small enough for the kernels' 32-bit per-row offsets within a 64-row tile.
bool strides_ok(const int64_t* st, bool o_bf16) {
  for (int t = 0; t < 4; ++t) {
    const int64_t unit = (t == 3 && !o_bf16) ? 4 : 8;  // elements per 16 bytes
    for (int a = 0; a < 3; ++a) {
      const int64_t x = st[3 * t + a];
      if (x < 0 || x % unit != 0) return false;
    }
    if (t < 3 && st[3 * t + 2] >= (int64_t(1) << 24)) return false;
  }
  return true;
}

int check_ex_args(const void* q, const void* k, const void* v, const void* o, int out_dtype,
                  const float* lse, const int64_t* strides, int B, int H, int S, int D,
                  float scale) {
  if (!q || !k || !v || !o || !strides) return DITATTN_EINVAL;
  if (out_dtype != DITATTN_OUT_F32 && out_dtype != DITATTN_OUT_BF16) return DITATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DITATTN_EINVAL;
  if (o == q || o == k || o == v) return DITATTN_EINVAL;
  if (lse && (!aligned(lse, 4) || static_cast<const void*>(lse) == o ||
              static_cast<const void*>(lse) == q || static_cast<const void*>(lse) == k ||
              static_cast<const void*>(lse) == v))
    return DITATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return DITATTN_EINVAL;
  const int st = check_attn_shape(B, H, S, D);
  if (st != DITATTN_OK) return st;
  if (!strides_ok(strides, out_dtype == DITATTN_OUT_BF16)) return DITATTN_EINVAL;
  return DITATTN_OK;
}

ditattn::AttnCall make_call(const void* q, const void* k, const void* v, void* o, bool o_bf16,
                            float* lse, const int64_t* st, int B, int H, int S, int D,
                            float scale) {
  ditattn::AttnCall ac;
  ac.q = q; ac.k = k; ac.v = v; ac.o = o; ac.o_bf16 = o_bf16; ac.lse = lse;
  ac.qs = {st[0], st[1], st[2]};
  ac.ks = {st[3], st[4], st[5]};
  ac.vs = {st[6], st[7], st[8]};
  ac.os = {st[9], st[10], st[11]};
  ac.B = B; ac.H = H; ac.S = S; ac.D = D; ac.scale = scale;
  ac.Sq = S;
  ac.tail = nullptr;
  ac.vt = nullptr;
  return ac;
}

// The attention launch's own scratch: the tail area, then (long sequences) the V^T tiles.
size_t attn_scratch_bytes(int B, int H, int S, int D) {
  return align_up(ditattn::attn_tail_bytes(S, D), kSegAlign) + ditattn::attn_vt_bytes(B, H, S, D);
}

void contiguous_strides(int H, int S, int D, int64_t st[12]) {
  for (int t = 0; t < 4; ++t) {
    st[3 * t] = (int64_t)H * S * D;
    st[3 * t + 1] = (int64_t)S * D;
    st[3 * t + 2] = D;
  }
}

enum Q8Mode { kQ8Int8, kQ8Fp8Qk, kQ8Fp8All };

// The int8 / fp8 paths after validation: workspace check, prepass, attention.
int q8_run(ditattn::AttnCall ac, Q8Mode mode, void* workspace, size_t workspace_bytes,
           hipStream_t s) {
  if (mode == kQ8Fp8All && ac.D != 128) return DITATTN_EUNSUPPORTED;
  const bool fp8 = mode != kQ8Int8;
  size_t off[9];
  const size_t need = mode == kQ8Fp8All ? attn_fp8_workspace_offsets(ac.B, ac.H, ac.S, ac.D, off)
                                        : attn_int8qk_workspace_offsets(ac.B, ac.H, ac.S, ac.D, off);
  if (!workspace || !aligned(workspace, kSegAlign) || workspace_bytes < need) return DITATTN_EWORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* k_mean = reinterpret_cast<float*>(ws + off[0]);
  float* q_scale = reinterpret_cast<float*>(ws + off[1]);
  float* k_scale = reinterpret_cast<float*>(ws + off[2]);
  int8_t* q_codes = reinterpret_cast<int8_t*>(ws + off[3]);
  int8_t* k_codes = reinterpret_cast<int8_t*>(ws + off[4]);
  double* partial = reinterpret_cast<double*>(ws + off[5]);
  // the scratch segment serves the attention launch too, after the prepass is done with it
  // (V^T tiles when V is bf16: not for fp8 for both products, which reads V codes)
  const size_t tail = ditattn::attn_tail_bytes(ac.S, ac.D);
  if (tail > 0) ac.tail = ws + off[5];
  if (mode != kQ8Fp8All && ditattn::attn_vt_bytes(ac.B, ac.H, ac.S, ac.D) > 0)
    ac.vt = ws + off[5] + align_up(tail, kSegAlign);
  const hipError_t e = ditattn::launch_prepass(ac.q, ac.qs, ac.k, ac.ks, k_mean, partial, q_codes,
                                               k_codes, q_scale, k_scale, ac.B, ac.H, ac.S, ac.D,
                                               fp8, s);
  if (e != hipSuccess) return DITATTN_EHIP;
  if (mode == kQ8Fp8All) {
    float* v_scale = reinterpret_cast<float*>(ws + off[6]);
    uint8_t* v_codes = ws + off[7];
    float* v_partial = reinterpret_cast<float*>(ws + off[8]);
    const hipError_t ev = ditattn::launch_vquant(ac.v, ac.vs, v_scale, v_partial, v_codes, ac.B,
                                                 ac.H, ac.S, ac.D, s);
    if (ev != hipSuccess) return DITATTN_EHIP;
    return status_of(ditattn::launch_attn_fp8_all(ac, reinterpret_cast<const uint8_t*>(q_codes),
                                                  reinterpret_cast<const uint8_t*>(k_codes), v_codes,
                                                  q_scale, k_scale, v_scale, s));
  }
  if (fp8)
    return status_of(ditattn::launch_attn_fp8(ac, reinterpret_cast<const uint8_t*>(q_codes),
                                              reinterpret_cast<const uint8_t*>(k_codes), q_scale,
                                              k_scale, s));
  return status_of(ditattn::launch_attn_int8(ac, q_codes, k_codes, q_scale, k_scale, s));
}

// Elementwise bf16 calls: out may be a or b exactly, but must not partly overlap either.
int check_elementwise(const void* a, const void* b, const void* out, int64_t n) {
  if (!a || !b || !out || n < 1) return DITATTN_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 16)) return DITATTN_EINVAL;
  if (n > (INT64_MAX / 2)) return DITATTN_EINVAL;
  const uintptr_t bytes = (uintptr_t)n * 2;
  auto partly = [&](const void* x) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(out), q = reinterpret_cast<uintptr_t>(x);
    return p != q && p < q + bytes && q < p + bytes;
  };
  if (partly(a) || partly(b)) return DITATTN_EINVAL;
  return DITATTN_OK;
}

}  // namespace

extern "C" {

const char* ditattn_status_string(int status) {
  switch (status) {
    case DITATTN_OK: return "ok";
    case DITATTN_EINVAL: return "invalid argument (null/misaligned pointer, size < 1, or bad scale)";
    case DITATTN_EUNSUPPORTED: return "unsupported head dimension (D must be 64 or 128)";
    case DITATTN_EWORKSPACE: return "workspace missing, misaligned or too small";
    case DITATTN_EHIP: return "HIP runtime error on kernel launch";
    default: return "unknown status";
  }
}

int attn_fwd_bf16(const void* q, const void* k, const void* v, float* o, int B, int H, int S,
                  int D, float scale, void* stream) {
  const int st = check_attn_args(q, k, v, o, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  int64_t strides[12];
  contiguous_strides(H, S, D, strides);
  return status_of(ditattn::launch_attn_bf16(
      make_call(q, k, v, o, false, nullptr, strides, B, H, S, D, scale),
      static_cast<hipStream_t>(stream)));
}

int attn_fwd_bf16_ex(const void* q, const void* k, const void* v, void* o, int out_dtype,
                     float* lse, const int64_t* strides, int B, int H, int S, int D, float scale,
                     void* stream) {
  const int st = check_ex_args(q, k, v, o, out_dtype, lse, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  return status_of(ditattn::launch_attn_bf16(
      make_call(q, k, v, o, out_dtype == DITATTN_OUT_BF16, lse, strides, B, H, S, D, scale),
      static_cast<hipStream_t>(stream)));
}

size_t attn_bf16_workspace_bytes(int B, int H, int S, int D) {
  if (check_attn_shape(B, H, S, D) != DITATTN_OK) return 0;
  return std::max(attn_scratch_bytes(B, H, S, D), kSegAlign);
}

int attn_fwd_bf16_ws(const void* q, const void* k, const void* v, void* o, int out_dtype,
                     float* lse, const int64_t* strides, int B, int H, int S, int D, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ex_args(q, k, v, o, out_dtype, lse, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  if (!workspace || !aligned(workspace, kSegAlign) ||
      workspace_bytes < attn_bf16_workspace_bytes(B, H, S, D))
    return DITATTN_EWORKSPACE;
  ditattn::AttnCall ac =
      make_call(q, k, v, o, out_dtype == DITATTN_OUT_BF16, lse, strides, B, H, S, D, scale);
  uint8_t* const ws = static_cast<uint8_t*>(workspace);
  const size_t tail = ditattn::attn_tail_bytes(S, D);
  if (tail > 0) ac.tail = ws;
  if (ditattn::attn_vt_bytes(B, H, S, D) > 0) ac.vt = ws + align_up(tail, kSegAlign);
  return status_of(ditattn::launch_attn_bf16(ac, static_cast<hipStream_t>(stream)));
}

size_t attn_int8qk_workspace_offsets(int B, int H, int S, int D, size_t offsets[6]) {
  if (check_attn_shape(B, H, S, D) != DITATTN_OK) return 0;
  const size_t bh = (size_t)B * (size_t)H;
  const size_t sizes[6] = {
      bh * D * sizeof(float),                               // k_mean
      bh * (size_t)((S + 127) / 128) * sizeof(float),       // q_scale
      bh * (size_t)((S + 63) / 64) * sizeof(float),         // k_scale
      bh * (size_t)S * D,                                   // q_codes
      bh * (size_t)S * D,                                   // k_codes
      // mean partials, then (once the codes are formed) the attention's scratch
      std::max(bh * (size_t)ditattn::kmean_chunks(B, H, S) * D * 2 * sizeof(double),
               attn_scratch_bytes(B, H, S, D)),
  };
  size_t off = 0;
  for (int i = 0; i < 6; ++i) {
    if (offsets) offsets[i] = off;
    off = align_up(off + sizes[i], kSegAlign);
  }
  return off;
}

size_t attn_int8qk_workspace_bytes(int B, int H, int S, int D) {
  return attn_int8qk_workspace_offsets(B, H, S, D, nullptr);
}

int attn_fwd_int8qk(const void* q, const void* k, const void* v, float* o, int B, int H, int S,
                    int D, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_attn_args(q, k, v, o, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  int64_t strides[12];
  contiguous_strides(H, S, D, strides);
  return q8_run(make_call(q, k, v, o, false, nullptr, strides, B, H, S, D, scale), kQ8Int8,
                workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int attn_fwd_int8qk_ex(const void* q, const void* k, const void* v, void* o, int out_dtype,
                       float* lse, const int64_t* strides, int B, int H, int S, int D,
                       float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ex_args(q, k, v, o, out_dtype, lse, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  return q8_run(
      make_call(q, k, v, o, out_dtype == DITATTN_OUT_BF16, lse, strides, B, H, S, D, scale), kQ8Int8,
      workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int attn_fwd_fp8qk(const void* q, const void* k, const void* v, float* o, int B, int H, int S,
                   int D, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_attn_args(q, k, v, o, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  int64_t strides[12];
  contiguous_strides(H, S, D, strides);
  return q8_run(make_call(q, k, v, o, false, nullptr, strides, B, H, S, D, scale), kQ8Fp8Qk,
                workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int attn_fwd_fp8qk_ex(const void* q, const void* k, const void* v, void* o, int out_dtype,
                      float* lse, const int64_t* strides, int B, int H, int S, int D, float scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ex_args(q, k, v, o, out_dtype, lse, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  return q8_run(
      make_call(q, k, v, o, out_dtype == DITATTN_OUT_BF16, lse, strides, B, H, S, D, scale), kQ8Fp8Qk,
      workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t attn_fp8_workspace_offsets(int B, int H, int S, int D, size_t offsets[9]) {
  size_t off6[6];
  const size_t base = attn_int8qk_workspace_offsets(B, H, S, D, off6);
  if (base == 0) return 0;
  const size_t bh = (size_t)B * (size_t)H;
  const size_t sizes[3] = {
      bh * D * sizeof(float),                                             // v_scale
      bh * (size_t)S * D,                                                 // v_codes
      bh * (size_t)ditattn::kmean_chunks(B, H, S) * D * sizeof(float),    // amax partials
  };
  size_t off = base;
  if (offsets)
    for (int i = 0; i < 6; ++i) offsets[i] = off6[i];
  for (int i = 0; i < 3; ++i) {
    if (offsets) offsets[6 + i] = off;
    off = align_up(off + sizes[i], kSegAlign);
  }
  return off;
}

size_t attn_fp8_workspace_bytes(int B, int H, int S, int D) {
  return attn_fp8_workspace_offsets(B, H, S, D, nullptr);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, float* o, int B, int H, int S, int D,
                 float scale, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_attn_args(q, k, v, o, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  int64_t strides[12];
  contiguous_strides(H, S, D, strides);
  return q8_run(make_call(q, k, v, o, false, nullptr, strides, B, H, S, D, scale), kQ8Fp8All,
                workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int attn_fwd_fp8_ex(const void* q, const void* k, const void* v, void* o, int out_dtype,
                    float* lse, const int64_t* strides, int B, int H, int S, int D, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ex_args(q, k, v, o, out_dtype, lse, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  return q8_run(
      make_call(q, k, v, o, out_dtype == DITATTN_OUT_BF16, lse, strides, B, H, S, D, scale), kQ8Fp8All,
      workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

size_t resid_rel_l1_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  return (size_t)ditattn::rel_l1_blocks(n) * 2 * sizeof(double);
}

int resid_rel_l1(const void* a, const void* b, int64_t n, float* out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (!a || !b || !out || n < 1) return DITATTN_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 4)) return DITATTN_EINVAL;
  if (!workspace || !aligned(workspace, 8) || workspace_bytes < resid_rel_l1_workspace_bytes(n))
    return DITATTN_EWORKSPACE;
  return status_of(ditattn::launch_rel_l1(a, b, n, out, static_cast<double*>(workspace),
                                          static_cast<hipStream_t>(stream)));
}

int resid_rel_l1_noalloc(const void* a, const void* b, int64_t n, float* out, void* stream) {
  if (!a || !b || !out || n < 1) return DITATTN_EINVAL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(out, 4)) return DITATTN_EINVAL;
  if ((size_t)ditattn::rel_l1_blocks(n) > ditattn::rel_l1_static_pairs()) return DITATTN_EWORKSPACE;
  return status_of(ditattn::launch_rel_l1_static(a, b, n, out, static_cast<hipStream_t>(stream)));
}

int attn_quant_probe_splits(int B, int H, int S, int D, int n_rows) {
  if (check_attn_shape(B, H, S, D) != DITATTN_OK || n_rows < 1 || n_rows > S) return 0;
  return ditattn::probe_chunks(B, H, S, n_rows).ns;
}

size_t attn_quant_probe_workspace_bytes(int B, int H, int S, int D, int n_rows) {
  if (check_attn_shape(B, H, S, D) != DITATTN_OK || n_rows < 1 || n_rows > S) return 0;
  const size_t ns = (size_t)ditattn::probe_chunks(B, H, S, n_rows).ns + 1;  // + the tail
  const size_t rows = (size_t)B * H * n_rows;
  return align_up(ns * rows * D * sizeof(float), kSegAlign) +
         align_up(ns * rows * sizeof(float), kSegAlign) +
         align_up((size_t)B * H * ditattn::probe_row_groups(n_rows) * 2 * sizeof(double), kSegAlign);
}

int attn_quant_probe(const void* q, const void* k, const void* v, const void* o_q, int o_q_dtype,
                     const int64_t* strides, int B, int H, int S, int D, float scale, int n_rows,
                     float* err, void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_ex_args(q, k, v, o_q, o_q_dtype, nullptr, strides, B, H, S, D, scale);
  if (st != DITATTN_OK) return st;
  if (n_rows < 1 || n_rows > S || !err || !aligned(err, 4)) return DITATTN_EINVAL;
  // the sampled rows are a strided view of q: its token stride times S / n_rows
  if (strides[2] * (S / n_rows) >= (int64_t(1) << 24)) return DITATTN_EINVAL;
  const size_t need = attn_quant_probe_workspace_bytes(B, H, S, D, n_rows);
  if (!workspace || !aligned(workspace, kSegAlign) || workspace_bytes < need) return DITATTN_EWORKSPACE;
  const size_t ns = (size_t)ditattn::probe_chunks(B, H, S, n_rows).ns + 1;
  const size_t rows = (size_t)B * H * n_rows;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* part = reinterpret_cast<float*>(ws);
  float* lse = reinterpret_cast<float*>(ws + align_up(ns * rows * D * sizeof(float), kSegAlign));
  double* sums = reinterpret_cast<double*>(reinterpret_cast<uint8_t*>(lse) +
                                           align_up(ns * rows * sizeof(float), kSegAlign));
  ditattn::AttnCall base = make_call(q, k, v, nullptr, false, nullptr, strides, B, H, S, D, scale);
  return status_of(ditattn::launch_quant_probe(base, o_q, o_q_dtype == DITATTN_OUT_BF16,
                                               base.os, n_rows, err, part, lse, sums,
                                               static_cast<hipStream_t>(stream)));
}

int fbcache_decide(const void* resid, const void* prev_resid, int64_t n,
                   const ditattn_fbcache_config* cfg, ditattn_fbcache_state* state,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!resid || !cfg || !state || n < 1) return DITATTN_EINVAL;
  if (!aligned(resid, 16) || !aligned(state, 4)) return DITATTN_EINVAL;
  if (prev_resid && !aligned(prev_resid, 16)) return DITATTN_EINVAL;
  const ditattn_fbcache_config c = *cfg;
  if (!isfinite(c.residual_diff_threshold) || c.residual_diff_threshold < 0.f) return DITATTN_EINVAL;
  if (c.max_warmup_steps < 0 || c.max_cached_steps < -1 || c.max_continuous_cached_steps < -1)
    return DITATTN_EINVAL;
  if (prev_resid && (!workspace || !aligned(workspace, 8) ||
                     workspace_bytes < resid_rel_l1_workspace_bytes(n)))
    return DITATTN_EWORKSPACE;
  return status_of(ditattn::launch_fbcache_decide(resid, prev_resid, n, c, state,
                                                  static_cast<double*>(workspace),
                                                  static_cast<hipStream_t>(stream)));
}

int ditattn_mfma_probe(int dtype, int random_operands, int iters, int64_t* clocks, void* stream) {
  if ((dtype != 0 && dtype != 1) || (random_operands != 0 && random_operands != 1)) return DITATTN_EINVAL;
  if (iters < 1 || !clocks || !aligned(clocks, 8)) return DITATTN_EINVAL;
  return status_of(ditattn::launch_mfma_probe(dtype == 1, random_operands == 1, iters, clocks,
                                              static_cast<hipStream_t>(stream)));
}

int resid_add(const void* a, const void* b, void* out, int64_t n, void* stream) {
  const int st = check_elementwise(a, b, out, n);
  if (st != DITATTN_OK) return st;
  return status_of(ditattn::launch_resid_addsub(a, b, out, n, false, static_cast<hipStream_t>(stream)));
}

int resid_sub(const void* a, const void* b, void* out, int64_t n, void* stream) {
  const int st = check_elementwise(a, b, out, n);
  if (st != DITATTN_OK) return st;
  return status_of(ditattn::launch_resid_addsub(a, b, out, n, true, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
