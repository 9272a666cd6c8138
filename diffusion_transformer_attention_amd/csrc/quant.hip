// Prepass of the int8-QK and fp8-QK attention for gfx950: K channel mean and per-block
// 8-bit codes.
//
// 8-bit attention (SageAttention) is the backend the "TMAP image-to-video inference
// acceleration" page adopts (section on combining with the quantized attention operator);
// its operator-details section reports that an all-zero group gives a zero scale, a division
// by zero and NaN outputs, which the scale rule below guards against.
//
// Contract implemented here (bit-exact, so the codes can be compared exactly):
//   k_mean[b,h,d] = fp32( fl64(exact sum_s K[b,h,s,d]) / S )
//   Ks            = fp32(K) - k_mean                      (one fp32 subtraction)
//   per block     amax = max |x|; scale = amax / 127 (IEEE fp32 division), 1.0 if amax == 0
//   code          = clamp(rint(x / scale), -127, 127)    (IEEE division, ties to even)
// fp8 e4m3 codes instead (QK on the fp8 matrix cores; the pages use fp8 for linear layers and
// 8-bit attention): scale = amax / 448 (the largest finite e4m3 value), code = x / scale
// clamped to [-448, 448] and rounded once to e4m3 (nearest, ties to even).
// Q blocks are 128 tokens and K blocks 64 tokens of one (b, h); a tail block covers only the
// valid tokens.  These kernels are bound by HBM bandwidth: every byte is read once (K twice:
// once for the mean, once for the codes) and every code written once, with 16-byte accesses.
// Three launches: the mean's partial sums together with the Q blocks (which do not need the
// mean), the mean itself, then the K blocks.
#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kThreads = 256;

// ---- K channel mean: exact double-double partial sums over token chunks ------------------
template <int D>
__device__ __forceinline__ void kmean_partial(const uint16_t* __restrict__ k, Strides ks, int H,
                                              double* __restrict__ partial, int S, int nch,
                                              int rows_per, int id) {
  constexpr int TPR = D / 8;             // threads per token row (8 channels each)
  constexpr int RPP = kThreads / TPR;    // rows per pass
  __shared__ double red_hi[kThreads][8];
  __shared__ double red_lo[kThreads][8];

  const int bh = id / nch;
  const int chunk = id - bh * nch;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  const int r0 = chunk * rows_per;
  const int r1 = min(S, r0 + rows_per);
  const uint16_t* kh = k + (bh / H) * ks.b + (bh % H) * ks.h;

  DDSum acc[8];
  auto add_row = [&](const u32x4& x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w].add((double)bf16lo(x[w]));
      acc[2 * w + 1].add((double)bf16hi(x[w]));
    }
  };
  // eight rows' loads in flight before their (long, dependent) double-double additions
  constexpr int U = 8;
  int row = r0 + rg;
  for (; row + (U - 1) * RPP < r1; row += U * RPP) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = *reinterpret_cast<const u32x4*>(kh + (int64_t)(row + u * RPP) * ks.s + cg * 8);
#pragma unroll
    for (int u = 0; u < U; ++u) add_row(x[u]);
  }
  for (; row < r1; row += RPP) add_row(*reinterpret_cast<const u32x4*>(kh + (int64_t)row * ks.s + cg * 8));
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red_hi[tid][e] = acc[e].hi;
    red_lo[tid][e] = acc[e].lo;
  }
  __syncthreads();
  if (tid < D) {
    const int g = tid / 8, e = tid % 8;
    DDSum s;
    for (int r = 0; r < RPP; ++r) s.merge(red_hi[r * TPR + g][e], red_lo[r * TPR + g][e]);
    double* dst = partial + 2 * (((size_t)bh * nch + chunk) * D + tid);
    dst[0] = s.hi;
    dst[1] = s.lo;
  }
}

// D / 32 workgroups per (b, h), 32 channels each: 8 lanes per channel each merge every 8th
// chunk (loads four chunks ahead of the merges), then a fixed tree joins the lanes; the exact
// sum is divided by S in fp64 and rounded once.
constexpr int kMeanCh = 32;                  // channels per workgroup
constexpr int kMeanLanes = kThreads / kMeanCh;

template <int D>
__global__ __launch_bounds__(kThreads) void kmean_final_kernel(const double* __restrict__ partial,
                                                               float* __restrict__ k_mean, int S,
                                                               int nch) {
  __shared__ double sh[kThreads], sl[kThreads];
  const int bh = blockIdx.x / (D / kMeanCh);
  const int d = (blockIdx.x % (D / kMeanCh)) * kMeanCh + threadIdx.x % kMeanCh;
  const int tid = threadIdx.x;
  const int part = tid / kMeanCh;
  const double* p = partial + 2 * ((size_t)bh * nch * D + d);
  DDSum s;
  int c = part;
  for (; c + 3 * kMeanLanes < nch; c += 4 * kMeanLanes) {
    double x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u][0] = p[2 * (size_t)(c + u * kMeanLanes) * D];
      x[u][1] = p[2 * (size_t)(c + u * kMeanLanes) * D + 1];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s.merge(x[u][0], x[u][1]);
  }
  for (; c < nch; c += kMeanLanes) s.merge(p[2 * (size_t)c * D], p[2 * (size_t)c * D + 1]);
  sh[tid] = s.hi;
  sl[tid] = s.lo;
  __syncthreads();
#pragma unroll
  for (int w = kMeanLanes / 2; w >= 1; w >>= 1) {
    if (part < w) {
      DDSum t{sh[tid], sl[tid]};
      t.merge(sh[tid + w * kMeanCh], sl[tid + w * kMeanCh]);
      sh[tid] = t.hi;
      sl[tid] = t.lo;
    }
    __syncthreads();
  }
  // sh[tid] (part 0) is the exact channel sum rounded once to fp64
  if (part == 0) k_mean[(size_t)bh * D + d] = (float)(sh[tid] / (double)S);
}

// ---- per-block quantization --------------------------------------------------------------
// One block of BT tokens of (b, h) = (bh / H, bh % H): x is read through its strides, the
// codes are written to the contiguous [B, H, S, D] buffer.
template <int D, int BT, bool SMOOTH, bool FP8>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ x, Strides xs, int H,
                                            const float* __restrict__ mean,
                                            int8_t* __restrict__ codes, float* __restrict__ scale_out,
                                            int S, int bh, int blk) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per token row
  constexpr int NC = (BT * CPR) / kThreads;        // chunks per thread
  static_assert(NC >= 1 && (BT * CPR) % kThreads == 0, "block shape");
  __shared__ float wmax[kThreads / 64];

  const int tid = threadIdx.x;
  const int t0 = blk * BT;
  const int nt = min(BT, S - t0);
  const size_t base = ((size_t)bh * S + t0) * D;                            // codes
  const uint16_t* xrow0 = x + (bh / H) * xs.b + (bh % H) * xs.h + (int64_t)t0 * xs.s;

  float v[NC][8];
  float amax = 0.f;
#pragma unroll
  for (int r = 0; r < NC; ++r) {
    const int id = tid + r * kThreads;
    const int tok = id / CPR, ch = id % CPR;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (tok < nt) w = *reinterpret_cast<const u32x4*>(xrow0 + (int64_t)tok * xs.s + ch * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[r][2 * e] = bf16lo(w[e]);
      v[r][2 * e + 1] = bf16hi(w[e]);
    }
    if constexpr (SMOOTH) {
      const f32x4 m0 = *reinterpret_cast<const f32x4*>(mean + (size_t)bh * D + ch * 8);
      const f32x4 m1 = *reinterpret_cast<const f32x4*>(mean + (size_t)bh * D + ch * 8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[r][e] = v[r][e] - m0[e];
        v[r][4 + e] = v[r][4 + e] - m1[e];
      }
    }
    if (tok < nt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[r][e]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  // the largest code: 127 (int8) or 448 (the largest finite fp8 e4m3 value)
  const float scale = (amax == 0.f) ? 1.0f : amax / (FP8 ? 448.0f : 127.0f);
  if (tid == 0) *scale_out = scale;
  // fl32(x / scale) is computed as fl32(fl64(x * fl64(1 / scale))), which is the same value
  // for every fp32 x and scale: the fp64 product is within 2^-52 (relative) of x / scale, while
  // a quotient of two 24-bit significands is either an fp32 rounding midpoint exactly (which
  // needs 25 significant bits, so never) or at least 2^-49 away from every midpoint.  Zero,
  // infinite and NaN operands give the same special values both ways.
  const double rinv = 1.0 / (double)scale;

#pragma unroll
  for (int r = 0; r < NC; ++r) {
    const int id = tid + r * kThreads;
    const int tok = id / CPR, ch = id % CPR;
    if (tok >= nt) continue;
    uint32_t packed[2] = {0u, 0u};
    if constexpr (FP8) {
      // x / scale (|x / scale| <= 448 up to one rounding, clamped), then one rounding to e4m3,
      // nearest even (v_cvt_pk_fp8_f32); fp32 first is innocuous (24 >= 2 * 4 + 2 bits)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        float qv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qv[e] = fminf(fmaxf((float)((double)v[r][4 * w + e] * rinv), -448.f), 448.f);
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], word, true);
        packed[w] = (uint32_t)word;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qv = rintf((float)((double)v[r][e] * rinv));
        qv = fminf(fmaxf(qv, -127.f), 127.f);
        packed[e >> 2] |= ((uint32_t)(uint8_t)(int8_t)(int)qv) << (8 * (e & 3));
      }
    }
    *reinterpret_cast<u32x2*>(codes + base + (size_t)tok * D + ch * 8) = u32x2{packed[0], packed[1]};
  }
}

// First pass of the prepass: the K-mean partial sums (ids below BH * nch) and, independent of
// the mean, the Q blocks (the remaining ids) in one launch.
template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void kmean_partial_quant_q_kernel(
    const uint16_t* __restrict__ q, Strides qs, const uint16_t* __restrict__ k, Strides ks, int H,
    double* __restrict__ partial, int8_t* __restrict__ q_codes, float* __restrict__ q_scale, int S,
    int BH, int nch, int rows_per, int nqb) {
  const int id = blockIdx.x;
  if (id < BH * nch) {
    kmean_partial<D>(k, ks, H, partial, S, nch, rows_per, id);
  } else {
    const int j = id - BH * nch;
    const int bh = j / nqb, blk = j - bh * nqb;
    quant_block<D, 128, false, FP8>(q, qs, H, nullptr, q_codes, q_scale + (size_t)bh * nqb + blk, S, bh,
                               blk);
  }
}

// Last pass: the K blocks, smoothed by the finished mean.
template <int D, bool FP8>
__global__ __launch_bounds__(kThreads) void quant_k_kernel(const uint16_t* __restrict__ k,
                                                           Strides ks, int H,
                                                           const float* __restrict__ k_mean,
                                                           int8_t* __restrict__ k_codes,
                                                           float* __restrict__ k_scale, int S,
                                                           int nkb) {
  const int bh = blockIdx.x / nkb, blk = blockIdx.x - bh * nkb;
  quant_block<D, 64, true, FP8>(k, ks, H, k_mean, k_codes, k_scale + (size_t)bh * nkb + blk, S, bh, blk);
}

// ---- fp8 V: per-channel amax over all tokens, then e4m3 codes ---------------------------
// Partial channel maxima of |V| over one token chunk (id = bh * nch + chunk): D / 8 threads per
// row read 16 bytes each, every max is exact, so chunking changes nothing.
template <int D>
__global__ __launch_bounds__(kThreads) void vmax_partial_kernel(const uint16_t* __restrict__ v,
                                                                Strides vs, int H,
                                                                float* __restrict__ partial, int S,
                                                                int nch, int rows_per) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  __shared__ float red[kThreads][8];
  const int id = blockIdx.x;
  const int bh = id / nch, chunk = id - bh * nch;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  const int r0 = chunk * rows_per;
  const int r1 = min(S, r0 + rows_per);
  const uint16_t* vh = v + (bh / H) * vs.b + (bh % H) * vs.h;
  float mx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  int row = r0 + rg;
  auto take = [&](const u32x4& x) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mx[2 * w] = fmaxf(mx[2 * w], fabsf(bf16lo(x[w])));
      mx[2 * w + 1] = fmaxf(mx[2 * w + 1], fabsf(bf16hi(x[w])));
    }
  };
  for (; row + (U - 1) * RPP < r1; row += U * RPP) {
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = *reinterpret_cast<const u32x4*>(vh + (int64_t)(row + u * RPP) * vs.s + cg * 8);
#pragma unroll
    for (int u = 0; u < U; ++u) take(x[u]);
  }
  for (; row < r1; row += RPP) take(*reinterpret_cast<const u32x4*>(vh + (int64_t)row * vs.s + cg * 8));
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tid][e] = mx[e];
  __syncthreads();
  if (tid < D) {
    const int g = tid / 8, e = tid % 8;
    float m = 0.f;
    for (int r = 0; r < RPP; ++r) m = fmaxf(m, red[r * TPR + g][e]);
    partial[((size_t)bh * nch + chunk) * D + tid] = m;
  }
}

// One workgroup per (b, h): the channel maxima over all chunks and the scales amax / 448.
template <int D>
__global__ __launch_bounds__(kThreads) void vscale_kernel(const float* __restrict__ partial,
                                                          float* __restrict__ v_scale, int nch) {
  const int bh = blockIdx.x;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float m = 0.f;
    for (int c = 0; c < nch; ++c) m = fmaxf(m, partial[((size_t)bh * nch + c) * D + d]);
    v_scale[(size_t)bh * D + d] = (m == 0.f) ? 1.0f : m / 448.0f;
  }
}

// e4m3 codes of one block of 64 tokens of (b, h) = (bh / H, bh % H), contiguous output.
template <int D>
__global__ __launch_bounds__(kThreads) void quant_v_kernel(const uint16_t* __restrict__ v, Strides vs,
                                                           int H, const float* __restrict__ v_scale,
                                                           uint8_t* __restrict__ codes, int S,
                                                           int nvb) {
  constexpr int CPR = D / 8;
  constexpr int BT = 64;
  constexpr int NC = (BT * CPR) / kThreads;
  static_assert(NC >= 1 && (BT * CPR) % kThreads == 0, "block shape");
  const int bh = blockIdx.x / nvb, blk = blockIdx.x - bh * nvb;
  const int tid = threadIdx.x;
  const int t0 = blk * BT;
  const int nt = min(BT, S - t0);
  const uint16_t* vrow0 = v + (bh / H) * vs.b + (bh % H) * vs.h + (int64_t)t0 * vs.s;
  const size_t base = ((size_t)bh * S + t0) * D;
#pragma unroll
  for (int r = 0; r < NC; ++r) {
    const int id = tid + r * kThreads;
    const int tok = id / CPR, ch = id % CPR;
    if (tok >= nt) continue;
    const u32x4 w = *reinterpret_cast<const u32x4*>(vrow0 + (int64_t)tok * vs.s + ch * 8);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(v_scale + (size_t)bh * D + ch * 8);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(v_scale + (size_t)bh * D + ch * 8 + 4);
    float x[8], sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16lo(w[e]);
      x[2 * e + 1] = bf16hi(w[e]);
      sc[e] = s0[e];
      sc[4 + e] = s1[e];
    }
    uint32_t packed[2];
#pragma unroll
    for (int d2 = 0; d2 < 2; ++d2) {
      float qv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // fl32(x / scale) as fl32(x * fl64(1 / scale)) (the same value, see quant_block)
        const double rinv = 1.0 / (double)sc[4 * d2 + e];
        qv[e] = fminf(fmaxf((float)((double)x[4 * d2 + e] * rinv), -448.f), 448.f);
      }
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(qv[0], qv[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(qv[2], qv[3], word, true);
      packed[d2] = (uint32_t)word;
    }
    *reinterpret_cast<u32x2*>(codes + base + (size_t)tok * D + ch * 8) = u32x2{packed[0], packed[1]};
  }
}

}  // namespace

hipError_t launch_vquant(const void* v, Strides vs, float* v_scale, float* partial,
                         uint8_t* v_codes, int B, int H, int S, int D, hipStream_t stream) {
  if (D != 128) return hipErrorInvalidValue;
  const int BH = B * H;
  const int nch = kmean_chunks(B, H, S);
  const int rows_per = (S + nch - 1) / nch;
  const int nvb = (S + 63) / 64;
  const auto* vv = static_cast<const uint16_t*>(v);
  hipLaunchKernelGGL(vmax_partial_kernel<128>, dim3((unsigned)((long long)BH * nch)), dim3(kThreads),
                     0, stream, vv, vs, H, partial, S, nch, rows_per);
  hipLaunchKernelGGL(vscale_kernel<128>, dim3((unsigned)BH), dim3(kThreads), 0, stream, partial,
                     v_scale, nch);
  hipLaunchKernelGGL(quant_v_kernel<128>, dim3((unsigned)((long long)BH * nvb)), dim3(kThreads), 0,
                     stream, vv, vs, H, v_scale, v_codes, S, nvb);
  return hipGetLastError();
}

int kmean_chunks(int B, int H, int S) {
  const long long bh = (long long)B * H;
  long long by_rows = (S + 127) / 128;
  long long by_grid = (2048 + bh - 1) / bh;
  long long n = by_rows < by_grid ? by_rows : by_grid;
  return (int)(n < 1 ? 1 : n);
}

template <int D, bool FP8>
hipError_t launch_prepass_d(const uint16_t* q, Strides qs, const uint16_t* k, Strides ks,
                            float* k_mean, double* partial, int8_t* q_codes, int8_t* k_codes,
                            float* q_scale, float* k_scale, int B, int H, int S, hipStream_t stream) {
  const int BH = B * H;
  const int nch = kmean_chunks(B, H, S);
  const int rows_per = (S + nch - 1) / nch;
  const int nqb = (S + 127) / 128, nkb = (S + 63) / 64;
  hipLaunchKernelGGL((kmean_partial_quant_q_kernel<D, FP8>),
                     dim3((unsigned)((long long)BH * (nch + nqb))), dim3(kThreads), 0, stream, q, qs,
                     k, ks, H, partial, q_codes, q_scale, S, BH, nch, rows_per, nqb);
  hipLaunchKernelGGL(kmean_final_kernel<D>, dim3((unsigned)(BH * (D / kMeanCh))), dim3(kThreads), 0,
                     stream, partial, k_mean, S, nch);
  hipLaunchKernelGGL((quant_k_kernel<D, FP8>), dim3((unsigned)((long long)BH * nkb)), dim3(kThreads),
                     0, stream, k, ks, H, k_mean, k_codes, k_scale, S, nkb);
  return hipGetLastError();
}

hipError_t launch_prepass(const void* q, Strides qs, const void* k, Strides ks, float* k_mean,
                          double* partial, int8_t* q_codes, int8_t* k_codes, float* q_scale,
                          float* k_scale, int B, int H, int S, int D, bool fp8, hipStream_t stream) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  if (D == 64) {
    if (fp8)
      return launch_prepass_d<64, true>(qq, qs, kk, ks, k_mean, partial, q_codes, k_codes, q_scale,
                                        k_scale, B, H, S, stream);
    return launch_prepass_d<64, false>(qq, qs, kk, ks, k_mean, partial, q_codes, k_codes, q_scale,
                                       k_scale, B, H, S, stream);
  }
  if (fp8)
    return launch_prepass_d<128, true>(qq, qs, kk, ks, k_mean, partial, q_codes, k_codes, q_scale,
                                       k_scale, B, H, S, stream);
  return launch_prepass_d<128, false>(qq, qs, kk, ks, k_mean, partial, q_codes, k_codes, q_scale,
                                      k_scale, B, H, S, stream);
}

}  // namespace ditattn
