// Quantization-error probe for gfx950: relative L2 distance of a quantized attention call's
// output from the bf16 path's output, on evenly spaced query rows.
//
// The "TMAP image-to-video inference acceleration" page (section on preserving video quality)
// keeps the attention layers whose quantized error is large in full precision; this measures
// that error for one call at a small fraction of its cost.  The bf16 attention of the sampled
// rows (step / 2 + i step, step = S / R: the middle row of each of R bins of step rows) runs
// as attn_fwd_kernel on a strided view of Q, with the keys split into chunks (a few hundred
// rows per head would otherwise fill only a few CUs); each chunk returns its partial output
// and log-sum-exp, and the kernels here merge the chunks (o = sum_c e^(lse_c - lse) o_c,
// lse = log sum_c e^lse_c) and reduce the squared differences in fp64: one workgroup per
// (b, h), then one workgroup for the total.
#include <math.h>

#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void block_sum2(double& x, double& y) {
  __shared__ double sx[kThreads / 64], sy[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    x += __shfl_xor(x, off, 64);
    y += __shfl_xor(y, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    sx[threadIdx.x >> 6] = x;
    sy[threadIdx.x >> 6] = y;
  }
  __syncthreads();
  x = ((sx[0] + sx[1]) + sx[2]) + sx[3];
  y = ((sy[0] + sy[1]) + sy[2]) + sy[3];
  __syncthreads();
}

// One workgroup per (b, h): merge the chunks of each sampled row and accumulate
// sum (o_q - o)^2 and sum o^2 over the row's D channels.
//   part  : fp32 [nsplit][B*H][R][D] chunk outputs;  lse : fp32 [nsplit][B*H][R]
//   o_q   : the quantized call's output (fp32 or bf16) at strides os
__global__ __launch_bounds__(kThreads) void probe_head_kernel(
    const float* __restrict__ part, const float* __restrict__ lse, int nsplit,
    const void* __restrict__ o_q, int o_bf16, Strides os, int H, int step, int R, int D,
    double* __restrict__ sums, float* __restrict__ err) {
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int BH = gridDim.x;
  double num = 0.0, den = 0.0;
  for (int e = threadIdx.x; e < R * D; e += kThreads) {
    const int i = e / D, d = e - i * D;
    // merge the key chunks of row i
    float m = -INFINITY;
    for (int c = 0; c < nsplit; ++c) m = fmaxf(m, lse[((size_t)c * BH + bh) * R + i]);
    double wsum = 0.0, acc = 0.0;
    for (int c = 0; c < nsplit; ++c) {
      const double w = exp((double)lse[((size_t)c * BH + bh) * R + i] - (double)m);
      wsum += w;
      acc += w * (double)part[(((size_t)c * BH + bh) * R + i) * D + d];
    }
    const double o = acc / wsum;
    const int64_t row = (int64_t)(step / 2) + (int64_t)i * step;
    const int64_t off = b * os.b + h * os.h + row * os.s + d;
    const double oq = o_bf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(o_q)[off] << 16)
                             : (double)static_cast<const float*>(o_q)[off];
    num += (oq - o) * (oq - o);
    den += o * o;
  }
  block_sum2(num, den);
  if (threadIdx.x == 0) {
    sums[2 * bh] = num;
    sums[2 * bh + 1] = den;
    err[1 + bh] = (float)sqrt(num / den);
  }
}

__global__ __launch_bounds__(kThreads) void probe_total_kernel(const double* __restrict__ sums,
                                                               int BH, float* __restrict__ err) {
  double num = 0.0, den = 0.0;
  for (int j = threadIdx.x; j < BH; j += kThreads) {
    num += sums[2 * j];
    den += sums[2 * j + 1];
  }
  block_sum2(num, den);
  if (threadIdx.x == 0) err[0] = (float)sqrt(num / den);
}

}  // namespace

int probe_splits(int B, int H, int S, int R) {
  const long long wg_rows = (long long)B * H * ((R + 255) / 256);  // workgroups per key chunk
  long long n = 256 / (wg_rows > 0 ? wg_rows : 1);
  const long long by_len = S / 1024;  // chunks of at least ~1024 keys
  if (n > by_len) n = by_len;
  if (n > 16) n = 16;
  if (n < 1) n = 1;
  return (int)n;
}

hipError_t launch_quant_probe(const AttnCall& base, const void* o_q, bool o_q_bf16, Strides oqs,
                              int R, float* err, float* part, float* lse, double* sums,
                              hipStream_t stream) {
  const int B = base.B, H = base.H, S = base.S, D = base.D;
  const int ns = probe_splits(B, H, S, R);
  const int step = S / R;
  // chunk c: keys [c L, min(S, (c + 1) L)), L a multiple of 64
  const int L = ((S + ns - 1) / ns + 63) / 64 * 64;
  for (int c = 0; c < ns; ++c) {
    const int k0 = c * L;
    if (k0 >= S) {
      // (cannot happen for the split counts above, but keep every chunk's output defined)
      return hipErrorInvalidValue;
    }
    AttnCall ac = base;
    // rows step/2 + i step of q: a view with that offset and token stride step * qs.s
    ac.q = static_cast<const uint16_t*>(base.q) + (int64_t)(step / 2) * base.qs.s;
    ac.qs.s = base.qs.s * step;
    ac.k = static_cast<const uint16_t*>(base.k) + k0 * base.ks.s;
    ac.v = static_cast<const uint16_t*>(base.v) + k0 * base.vs.s;
    ac.S = (S - k0 < L) ? S - k0 : L;
    ac.Sq = R;
    ac.o = part + (size_t)c * B * H * R * D;
    ac.o_bf16 = false;
    ac.os = {(int64_t)H * R * D, (int64_t)R * D, D};
    ac.lse = lse + (size_t)c * B * H * R;
    const hipError_t e = launch_attn_bf16(ac, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(probe_head_kernel, dim3((unsigned)(B * H)), dim3(kThreads), 0, stream, part,
                     lse, ns, o_q, o_q_bf16 ? 1 : 0, oqs, H, step, R, D, sums, err);
  hipLaunchKernelGGL(probe_total_kernel, dim3(1), dim3(kThreads), 0, stream, sums, B * H, err);
  return hipGetLastError();
}

}  // namespace ditattn
