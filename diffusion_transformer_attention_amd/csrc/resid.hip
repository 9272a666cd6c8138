// Residual arithmetic of First Block Cache for gfx950: out = bf16(a + b) or bf16(a - b).
//
// When a denoising step reuses the cache ("ParaAttention" page, First Block Cache section), its
// output is the first block's output plus the residual the remaining blocks added at the latest
// computed step; when it computes, that residual is formed as the final hidden states minus
// the first block's output.  Both are elementwise over the hidden states, bound by HBM
// bandwidth (6 bytes per element: two bf16 reads, one bf16 write).  A grid-stride loop over
// groups of 16-byte chunks, four per thread in flight, with nontemporal loads and stores
// (nothing is reread); at [118800, 3072] each workgroup takes one group (measured 6.4 TB/s
// against 5.0 for one contiguous range per workgroup).  The sum is formed in fp32 and rounded once to bf16 (nearest
// even); the fp32 rounding before it cannot change the result (24 >= 2 * 8 + 2 bits), so each
// value is the exact sum or difference rounded once.
#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kMaxBlocks = 65536;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool SUB>
__device__ __forceinline__ uint32_t addsub2(uint32_t a, uint32_t b) {
  const float lo = SUB ? bf16lo(a) - bf16lo(b) : bf16lo(a) + bf16lo(b);
  const float hi = SUB ? bf16hi(a) - bf16hi(b) : bf16hi(a) + bf16hi(b);
  const bf16x2_t r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

template <bool SUB>
__device__ __forceinline__ u32x4 addsub8(const u32x4& a, const u32x4& b) {
  return u32x4{addsub2<SUB>(a[0], b[0]), addsub2<SUB>(a[1], b[1]), addsub2<SUB>(a[2], b[2]),
               addsub2<SUB>(a[3], b[3])};
}

// (no __restrict__: out may be a or b itself; each element is read before its own store)
template <bool SUB>
__global__ __launch_bounds__(kThreads) void resid_addsub_kernel(const uint16_t* a, const uint16_t* b,
                                                                uint16_t* out, int64_t n) {
  const int64_t n8 = n >> 3;
  const u32x4* a8 = reinterpret_cast<const u32x4*>(a);
  const u32x4* b8 = reinterpret_cast<const u32x4*>(b);
  u32x4* o8 = reinterpret_cast<u32x4*>(out);
  // grid-stride over groups of kUnroll * kThreads chunks (one group per workgroup when the
  // grid is not capped)
  const int64_t step = (int64_t)gridDim.x * kUnroll * kThreads;
  int64_t i = (int64_t)blockIdx.x * kUnroll * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < n8; i += step) {
    u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      va[u] = __builtin_nontemporal_load(a8 + i + u * kThreads);
      vb[u] = __builtin_nontemporal_load(b8 + i + u * kThreads);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_nontemporal_store(addsub8<SUB>(va[u], vb[u]), o8 + i + u * kThreads);
  }
  for (; i < n8; i += kThreads)
    __builtin_nontemporal_store(
        addsub8<SUB>(__builtin_nontemporal_load(a8 + i), __builtin_nontemporal_load(b8 + i)), o8 + i);

  // the last n % 8 elements, one per thread of the first workgroup
  if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
    const int64_t e = (n8 << 3) + threadIdx.x;
    out[e] = (uint16_t)addsub2<SUB>(a[e], b[e]);
  }
}

}  // namespace

hipError_t launch_resid_addsub(const void* a, const void* b, void* out, int64_t n, bool sub,
                               hipStream_t stream) {
  const int64_t n8 = n >> 3;
  int64_t nb = (n8 + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (nb < 1) nb = 1;
  if (nb > kMaxBlocks) nb = kMaxBlocks;
  const auto* pa = static_cast<const uint16_t*>(a);
  const auto* pb = static_cast<const uint16_t*>(b);
  auto* po = static_cast<uint16_t*>(out);
  if (sub)
    hipLaunchKernelGGL(resid_addsub_kernel<true>, dim3((unsigned)nb), dim3(kThreads), 0, stream,
                       pa, pb, po, n);
  else
    hipLaunchKernelGGL(resid_addsub_kernel<false>, dim3((unsigned)nb), dim3(kThreads), 0, stream,
                       pa, pb, po, n);
  return hipGetLastError();
}

}  // namespace ditattn
