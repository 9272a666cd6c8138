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
// lse = log sum_c e^lse_c) and reduce the squared differences in fp64: one workgroup per eight
// sampled rows, then one workgroup for the per-head and overall totals.
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

constexpr int kRowsPerWG = 8;    // sampled rows per workgroup of the merge
constexpr int kMaxChunks = 17;   // probe_splits' 16 uniform chunks and the tail

// One workgroup per kRowsPerWG sampled rows of one (b, h): merge the key chunks of each row and
// accumulate sum (o_q - o)^2 and sum o^2 over those rows' D channels into sums[bh][g].
//   part  : fp32 [B][nslot][H][R][D] chunk outputs;  lse : fp32 [B][nslot][H][R]; chunks
//           0 .. nused-1 hold results
//   o_q   : the quantized call's output (fp32 or bf16) at strides os
__global__ __launch_bounds__(kThreads) void probe_rows_kernel(
    const float* __restrict__ part, const float* __restrict__ lse, int nslot, int nused,
    const void* __restrict__ o_q, int o_bf16, Strides os, int H, int step, int R, int D, int ngrp,
    double* __restrict__ sums) {
  __shared__ float wts[kRowsPerWG][kMaxChunks];   // normalised chunk weights of each row
  const int bh = blockIdx.x / ngrp, g = blockIdx.x - bh * ngrp;
  const int b = bh / H, h = bh - b * H;
  const int i0 = g * kRowsPerWG;
  const int nr = min(kRowsPerWG, R - i0);
  auto at = [&](int c, int i) { return ((size_t)(b * nslot + c) * H + h) * R + i; };
  if (threadIdx.x < nr) {
    // e^(lse_c - m) / sum_c e^(lse_c - m) in fp32: relative error ~1e-7, far below anything
    // an error estimate needs
    const int i = i0 + threadIdx.x;
    float m = -INFINITY;
    for (int c = 0; c < nused; ++c) m = fmaxf(m, lse[at(c, i)]);
    float w[kMaxChunks], sw = 0.f;
    for (int c = 0; c < nused; ++c) {
      w[c] = __expf(lse[at(c, i)] - m);
      sw += w[c];
    }
    for (int c = 0; c < nused; ++c) wts[threadIdx.x][c] = w[c] / sw;
  }
  __syncthreads();
  double num = 0.0, den = 0.0;
  for (int e = threadIdx.x; e < nr * D; e += kThreads) {
    const int r = e / D, d = e - r * D;
    const int i = i0 + r;
    double o = 0.0;
    for (int c = 0; c < nused; ++c) o += (double)wts[r][c] * (double)part[at(c, i) * D + d];
    const int64_t row = (int64_t)(step / 2) + (int64_t)i * step;
    const int64_t off = b * os.b + h * os.h + row * os.s + d;
    const double oq = o_bf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(o_q)[off] << 16)
                             : (double)static_cast<const float*>(o_q)[off];
    num += (oq - o) * (oq - o);
    den += o * o;
  }
  block_sum2(num, den);
  if (threadIdx.x == 0) {
    sums[2 * blockIdx.x] = num;
    sums[2 * blockIdx.x + 1] = den;
  }
}

// One workgroup: each head's sums over its row groups (err[1 + bh]), then all heads (err[0]).
__global__ __launch_bounds__(kThreads) void probe_total_kernel(const double* __restrict__ sums,
                                                               int BH, int ngrp,
                                                               float* __restrict__ err) {
  double num = 0.0, den = 0.0;
  for (int bh = threadIdx.x; bh < BH; bh += kThreads) {
    double hn = 0.0, hd = 0.0;
    for (int g = 0; g < ngrp; ++g) {
      hn += sums[2 * ((size_t)bh * ngrp + g)];
      hd += sums[2 * ((size_t)bh * ngrp + g) + 1];
    }
    err[1 + bh] = (float)sqrt(hn / hd);
    num += hn;
    den += hd;
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

int probe_row_groups(int R) { return (R + kRowsPerWG - 1) / kRowsPerWG; }

ProbeChunks probe_chunks(int B, int H, int S, int R) {
  ProbeChunks pc;
  pc.ns = probe_splits(B, H, S, R);
  pc.L = (S / pc.ns) / 64 * 64;
  if (pc.ns == 1 || pc.L == 0) {
    pc.ns = 1;
    pc.L = S;
  }
  pc.tail = S - pc.ns * pc.L;
  return pc;
}

hipError_t launch_quant_probe(const AttnCall& base, const void* o_q, bool o_q_bf16, Strides oqs,
                              int R, float* err, float* part, float* lse, double* sums,
                              hipStream_t stream) {
  const int B = base.B, H = base.H, S = base.S, D = base.D;
  const ProbeChunks pc = probe_chunks(B, H, S, R);
  const int nslot = pc.ns + 1;
  const int step = S / R;
  for (int b = 0; b < B; ++b) {
    // the uniform chunks of batch b in one launch: chunk c is virtual batch c, whose keys start
    // c L rows further on (batch stride L rows) and whose query rows are the same (stride 0)
    AttnCall ac = base;
    ac.B = pc.ns;
    ac.S = pc.L;
    ac.Sq = R;
    // sampled rows step/2 + i step: a view of q with that offset and token stride step rows
    ac.q = static_cast<const uint16_t*>(base.q) + b * base.qs.b + (int64_t)(step / 2) * base.qs.s;
    ac.qs = {0, base.qs.h, base.qs.s * step};
    ac.k = static_cast<const uint16_t*>(base.k) + b * base.ks.b;
    ac.ks = {(int64_t)pc.L * base.ks.s, base.ks.h, base.ks.s};
    ac.v = static_cast<const uint16_t*>(base.v) + b * base.vs.b;
    ac.vs = {(int64_t)pc.L * base.vs.s, base.vs.h, base.vs.s};
    ac.o = part + (size_t)b * nslot * H * R * D;
    ac.o_bf16 = false;
    ac.os = {(int64_t)H * R * D, (int64_t)R * D, D};
    ac.lse = lse + (size_t)b * nslot * H * R;  // [chunk][h][row] of batch b
    hipError_t e = launch_attn_bf16(ac, stream);
    if (e != hipSuccess) return e;
    if (pc.tail > 0) {
      // the remaining S - ns L keys as chunk ns
      AttnCall at = ac;
      at.B = 1;
      at.S = pc.tail;
      at.k = static_cast<const uint16_t*>(ac.k) + (int64_t)pc.ns * pc.L * base.ks.s;
      at.v = static_cast<const uint16_t*>(ac.v) + (int64_t)pc.ns * pc.L * base.vs.s;
      at.o = static_cast<float*>(ac.o) + (size_t)pc.ns * H * R * D;
      at.lse = ac.lse + (size_t)pc.ns * H * R;
      e = launch_attn_bf16(at, stream);
      if (e != hipSuccess) return e;
    }
  }
  const int ngrp = probe_row_groups(R);
  hipLaunchKernelGGL(probe_rows_kernel, dim3((unsigned)(B * H * ngrp)), dim3(kThreads), 0, stream,
                     part, lse, nslot, pc.ns + (pc.tail > 0 ? 1 : 0), o_q, o_q_bf16 ? 1 : 0, oqs,
                     H, step, R, D, ngrp, sums);
  hipLaunchKernelGGL(probe_total_kernel, dim3(1), dim3(kThreads), 0, stream, sums, B * H, ngrp, err);
  return hipGetLastError();
}

}  // namespace ditattn
