// Relative L1 distance of two bf16 residual tensors for gfx950: sum|a - b| / sum|b|.
//
// First Block Cache ("ParaAttention" page, First Block Cache section) skips the remaining
// transformer blocks of a denoising step when the first block's residual differs little from
// the previous step's; this is the difference it compares with its threshold.  The pass is
// bound by HBM bandwidth (4 bytes read per element, ~3 flops): a grid-stride loop over groups
// of 16-byte chunks (four per thread in flight, nontemporal loads; measured 7.0 TB/s against
// 6.5 for one contiguous range per workgroup with eight in flight), fp32 per-thread sums, an
// fp64 reduction per workgroup, and a one-workgroup fp64 finish in a fixed order (no atomics,
// so the result is deterministic).
//
// fbcache_decide runs the same pass and then, in the finishing workgroup, the cache decision
// of the step: reuse only past the warmup steps, with a difference below the threshold, and
// within the caps on cached and consecutively cached steps (DBCache parameters of the
// "Cache-DiT acceleration" page).  The decision and the counters stay in device memory.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kMaxBlocks = 4096;  // (16384 reads 0.5% faster but quadruples the finish)

__device__ __forceinline__ void accum8(const u32x4& a, const u32x4& b, float& num, float& den) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = bf16lo(a[w]), a1 = bf16hi(a[w]);
    const float b0 = bf16lo(b[w]), b1 = bf16hi(b[w]);
    num += fabsf(a0 - b0) + fabsf(a1 - b1);
    den += fabsf(b0) + fabsf(b1);
  }
}

// Sum of the nblocks (x, y) partial pairs over the workgroup's threads: each thread adds its
// strided share four loads at a time (independent, so they overlap), in a fixed order.
__device__ __forceinline__ void sum_partials(const double* __restrict__ partial, int nblocks,
                                             double& x, double& y) {
  double xs[4] = {0.0, 0.0, 0.0, 0.0}, ys[4] = {0.0, 0.0, 0.0, 0.0};
  int j = threadIdx.x;
  for (; j + 3 * kThreads < nblocks; j += 4 * kThreads) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      xs[u] += partial[2 * (j + u * kThreads)];
      ys[u] += partial[2 * (j + u * kThreads) + 1];
    }
  }
  for (int u = 0; j < nblocks; j += kThreads, ++u) {
    xs[u] += partial[2 * j];
    ys[u] += partial[2 * j + 1];
  }
  x = (xs[0] + xs[1]) + (xs[2] + xs[3]);
  y = (ys[0] + ys[1]) + (ys[2] + ys[3]);
}

__device__ __forceinline__ void block_reduce2(double& x, double& y) {
  __shared__ double sx[kThreads / 64], sy[kThreads / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    x += __shfl_xor(x, off, 64);
    y += __shfl_xor(y, off, 64);
  }
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) {
    sx[tid >> 6] = x;
    sy[tid >> 6] = y;
  }
  __syncthreads();
  x = ((sx[0] + sx[1]) + sx[2]) + sx[3];
  y = ((sy[0] + sy[1]) + sy[2]) + sy[3];
}

__global__ __launch_bounds__(kThreads) void rel_l1_partial_kernel(const uint16_t* __restrict__ a,
                                                                  const uint16_t* __restrict__ b,
                                                                  int64_t n, double* __restrict__ partial) {
  const int64_t n8 = n >> 3;  // whole 16-byte chunks
  const u32x4* a8 = reinterpret_cast<const u32x4*>(a);
  const u32x4* b8 = reinterpret_cast<const u32x4*>(b);
  // grid-stride over groups of kUnroll * kThreads chunks: at any moment the whole grid reads
  // one compact window of the tensors
  const int64_t step = (int64_t)gridDim.x * kUnroll * kThreads;
  float num = 0.f, den = 0.f;
  int64_t i = (int64_t)blockIdx.x * kUnroll * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n8; i += step) {
    u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      va[u] = __builtin_nontemporal_load(a8 + i + u * kThreads);
      vb[u] = __builtin_nontemporal_load(b8 + i + u * kThreads);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) accum8(va[u], vb[u], num, den);
  }
  for (; i < n8; i += kThreads)
    accum8(__builtin_nontemporal_load(a8 + i), __builtin_nontemporal_load(b8 + i), num, den);

  // the last n % 8 elements
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t e = (n8 << 3) + threadIdx.x;
    const float av = bf16lo(a[e]), bv = bf16lo(b[e]);
    num += fabsf(av - bv);
    den += fabsf(bv);
  }

  double x = num, y = den;
  block_reduce2(x, y);
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = x;
    partial[2 * blockIdx.x + 1] = y;
  }
}

__global__ __launch_bounds__(kThreads) void rel_l1_final_kernel(const double* __restrict__ partial,
                                                                int nblocks, float* __restrict__ out) {
  double x, y;
  sum_partials(partial, nblocks, x, y);
  block_reduce2(x, y);
  if (threadIdx.x == 0) {
    float r;
    if (y == 0.0)
      r = (x == 0.0) ? 0.f : INFINITY;
    else
      r = (float)(x / y);
    out[0] = r;
  }
}

// The same finish, followed by one First Block Cache decision on the state in device memory
// (thread 0 reads, decides and writes it back; calls on one state are ordered by the stream).
// nblocks == 0: there is no previous residual, so no difference and the step computes.
__global__ __launch_bounds__(kThreads) void fbcache_final_kernel(const double* __restrict__ partial,
                                                                 int nblocks,
                                                                 ditattn_fbcache_config cfg,
                                                                 ditattn_fbcache_state* state) {
  double x, y;
  sum_partials(partial, nblocks, x, y);
  block_reduce2(x, y);
  if (threadIdx.x == 0) {
    const bool has_prev = nblocks > 0;
    float r = __builtin_nanf("");
    if (has_prev) {
      if (y == 0.0)
        r = (x == 0.0) ? 0.f : INFINITY;
      else
        r = (float)(x / y);
    }
    ditattn_fbcache_state st = *state;
    // warmup, a difference below the threshold (false for NaN), and both caps
    bool use = st.steps >= cfg.max_warmup_steps && has_prev && r < cfg.residual_diff_threshold;
    if (cfg.max_cached_steps >= 0 && st.cached_steps >= cfg.max_cached_steps) use = false;
    if (cfg.max_continuous_cached_steps >= 0 &&
        st.continuous_cached_steps >= cfg.max_continuous_cached_steps)
      use = false;
    st.steps += 1;
    st.cached_steps += use ? 1 : 0;
    st.continuous_cached_steps = use ? st.continuous_cached_steps + 1 : 0;
    st.use_cache = use ? 1 : 0;
    st.diff = r;
    *state = st;
  }
}

}  // namespace

// ---- the allocation-free variant: partial sums in a static device array ---------------------
// For callers that cannot allocate device memory, the partial pairs go to this file-scope
// array: kMaxBlocks pairs (64 KiB), the most any n needs, one copy per GPU the library runs on,
// held until the process ends.  Its name is a host-side stand-in, not a device address: the
// address of each device's copy is looked up once (with that device current) and only that
// looked-up pointer reaches the kernels.  Every call on a GPU shares the array, so calls that
// overlap on one GPU race; nothing in it needs clearing, because the finishing kernel reads
// only the pairs the same call's partial kernel has just written.
static __device__ __align__(256) double scratch[2 * kMaxBlocks];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch[kMaxDevices] = {};

// This device's copy of `scratch`, the device being the one `stream` belongs to (the current
// device for the null stream).
hipError_t scratch_for(hipStream_t stream, double** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<double*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

size_t rel_l1_static_pairs() { return kMaxBlocks; }

hipError_t launch_rel_l1_static(const void* a, const void* b, int64_t n, float* out,
                                hipStream_t stream) {
  if ((size_t)rel_l1_blocks(n) > rel_l1_static_pairs()) return hipErrorInvalidValue;
  double* partial = nullptr;
  const hipError_t e = scratch_for(stream, &partial);
  if (e != hipSuccess) return e;
  return launch_rel_l1(a, b, n, out, partial, stream);
}

int rel_l1_blocks(int64_t n) {
  const int64_t n8 = n >> 3;
  int64_t nb = (n8 + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (nb < 1) nb = 1;
  if (nb > kMaxBlocks) nb = kMaxBlocks;
  return (int)nb;
}

hipError_t launch_rel_l1(const void* a, const void* b, int64_t n, float* out, double* partial,
                         hipStream_t stream) {
  const int nb = rel_l1_blocks(n);
  hipLaunchKernelGGL(rel_l1_partial_kernel, dim3(nb), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), n, partial);
  hipLaunchKernelGGL(rel_l1_final_kernel, dim3(1), dim3(kThreads), 0, stream, partial, nb, out);
  return hipGetLastError();
}

hipError_t launch_fbcache_decide(const void* resid, const void* prev_resid, int64_t n,
                                 const ditattn_fbcache_config& cfg, ditattn_fbcache_state* state,
                                 double* partial, hipStream_t stream) {
  int nb = 0;
  if (prev_resid != nullptr) {
    nb = rel_l1_blocks(n);
    hipLaunchKernelGGL(rel_l1_partial_kernel, dim3(nb), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(resid), static_cast<const uint16_t*>(prev_resid),
                       n, partial);
  }
  hipLaunchKernelGGL(fbcache_final_kernel, dim3(1), dim3(kThreads), 0, stream, partial, nb, cfg,
                     state);
  return hipGetLastError();
}

}  // namespace ditattn
