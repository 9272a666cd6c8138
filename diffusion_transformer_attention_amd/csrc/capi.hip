// C ABI of the library (declared in include/ditattn.h): argument validation, workspace
// layout and kernel launches on the caller's stream.  Validation never touches the HIP
// runtime, so a rejected call enqueues nothing and needs no GPU.
#include <math.h>
#include <stdint.h>

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
  return status_of(ditattn::launch_attn_bf16(q, k, v, o, B, H, S, D, scale,
                                             static_cast<hipStream_t>(stream)));
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
      bh * (size_t)ditattn::kmean_chunks(B, H, S) * D * 2 * sizeof(double),  // mean partials
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
  size_t off[6];
  const size_t need = attn_int8qk_workspace_offsets(B, H, S, D, off);
  if (!workspace || !aligned(workspace, kSegAlign) || workspace_bytes < need) return DITATTN_EWORKSPACE;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* k_mean = reinterpret_cast<float*>(ws + off[0]);
  float* q_scale = reinterpret_cast<float*>(ws + off[1]);
  float* k_scale = reinterpret_cast<float*>(ws + off[2]);
  int8_t* q_codes = reinterpret_cast<int8_t*>(ws + off[3]);
  int8_t* k_codes = reinterpret_cast<int8_t*>(ws + off[4]);
  double* partial = reinterpret_cast<double*>(ws + off[5]);
  hipStream_t s = static_cast<hipStream_t>(stream);

  const hipError_t e = ditattn::launch_prepass(q, k, k_mean, partial, q_codes, k_codes, q_scale,
                                               k_scale, B, H, S, D, s);
  if (e != hipSuccess) return DITATTN_EHIP;
  return status_of(ditattn::launch_attn_int8(q_codes, k_codes, v, o, q_scale, k_scale, B, H, S,
                                             D, scale, s));
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

}  // extern "C"
