// Calibration for measurement: the rate the matrix cores sustain when they do nothing else.
//
// Not part of the attention path.  Attention throughput is quoted against the nominal dense
// peaks (2.5 PFLOP/s bf16, 5.0 POP/s int8 at 2.4 GHz).  This kernel measures what the chip
// delivers on a stream of products alone: 1024 workgroups of 8 wavefronts (two per SIMD on
// every CU, four rounds), each wavefront issuing independent 32x32 products back to back with
// no other instruction in its loop.  With operands that differ between products and lanes
// (random values) the chip's power limit lowers the shader clock; with constant operands it
// runs near the rated clock.  Each workgroup records the shader clocks (s_memtime) and the
// 100 MHz reference clocks (s_memrealtime) it ran, so the caller can report the clock the
// products ran at next to the rate.
#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeWorkgroups = 1024;

__device__ __forceinline__ uint32_t xorshift(uint32_t& s) {
  s ^= s << 13;
  s ^= s >> 17;
  s ^= s << 5;
  return s;
}

template <bool INT8, bool RANDOM>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters,
                                                                  int64_t* __restrict__ clocks) {
  // four A and four B operands per lane; a product pairs A[m % 4] with B[(m / 2) % 4]
  bf16x8 a[4], b[4];
  i32x4 ia[4], ib[4];
  uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // values in [-2, 2) on a 2^-14 grid (RANDOM), else a fixed pattern
      a[r][i] = (__bf16)(RANDOM ? (float)(xorshift(h) & 0xFFFF) / 16384.0f - 2.0f : 0.25f * (i + 1));
      b[r][i] = (__bf16)(RANDOM ? (float)(xorshift(h) & 0xFFFF) / 16384.0f - 2.0f : 0.5f * (r + 1));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ia[r][i] = RANDOM ? (int)xorshift(h) : 0x01020304 * (r + 1);
      ib[r][i] = RANDOM ? (int)xorshift(h) : 0x05060708 + i;
    }
  }
  f32x16 acc[4] = {};
  i32x16 iacc[4] = {};
  const int64_t t0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if constexpr (INT8)
        iacc[m & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ia[m & 3], ib[(m >> 1) & 3], iacc[m & 3], 0, 0, 0);
      else
        acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m & 3], b[(m >> 1) & 3], acc[m & 3], 0, 0, 0);
    }
  }
  const int64_t t1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  // keep every product live: a value no accumulator can reach selects a store
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += INT8 ? (float)iacc[i][0] : acc[i][0];
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = (s == 1.0e30f) ? -1 : t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

int mfma_probe_workgroups() { return kProbeWorkgroups; }

hipError_t launch_mfma_probe(bool int8, bool random, int iters, int64_t* clocks, hipStream_t stream) {
  const dim3 grid(kProbeWorkgroups), block(kProbeThreads);
  if (int8) {
    if (random)
      hipLaunchKernelGGL((mfma_probe_kernel<true, true>), grid, block, 0, stream, iters, clocks);
    else
      hipLaunchKernelGGL((mfma_probe_kernel<true, false>), grid, block, 0, stream, iters, clocks);
  } else {
    if (random)
      hipLaunchKernelGGL((mfma_probe_kernel<false, true>), grid, block, 0, stream, iters, clocks);
    else
      hipLaunchKernelGGL((mfma_probe_kernel<false, false>), grid, block, 0, stream, iters, clocks);
  }
  return hipGetLastError();
}

}  // namespace ditattn
