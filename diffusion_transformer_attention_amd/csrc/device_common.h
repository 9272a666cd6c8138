// Device-side types and helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Exact widening of a bf16 bit pattern held in the low 16 bits.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
// Exact widening of a bf16 bit pattern held in the high 16 bits.
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to bf16 (nearest even) and return the bit pattern.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, b);
}

// Sum / max of a value held by lane l and lane l ^ 32 of a 64-wide wavefront.
// v_permlane32_swap(x, x) returns {x, x of lane l ^ 32} in some order on every lane.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int xor32_max_i32(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Knuth's TwoSum: a + b is represented exactly as s + e with s = fl(a + b), for any
// finite a, b (no ordering precondition).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// Exact accumulation of fp64 values into an unevaluated sum hi + lo with hi = fl(hi + lo).
// Every step is exact while the accumulated values span fewer than ~105 bits.
struct DDSum {
  double hi = 0.0, lo = 0.0;
  __device__ __forceinline__ void add(double x) {
    double s, e;
    two_sum(hi, x, s, e);
    double t = lo + e;
    two_sum(s, t, hi, lo);
  }
  __device__ __forceinline__ void merge(double ohi, double olo) {
    double s, e;
    two_sum(hi, ohi, s, e);
    double t = (lo + olo) + e;
    two_sum(s, t, hi, lo);
  }
};

}  // namespace ditattn
