// Non-causal multi-head attention forward for gfx950 (MI355X): bf16 and int8-QK variants.
//
// O = softmax(Q K^T * scale) V, computed blockwise on chip so the S x S score matrix never
// reaches HBM (the IO-aware tiling of the "Flash Attention 2 for Z-Image S3-DiT" page, method
// paragraph), with a streaming (online) softmax: a running row maximum m and row sum l,
// rescaled by 2^(m_old - m_new) whenever a new key tile raises the maximum.  The final
// division by l makes the result exact attention up to rounding.
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows of one (b, h)):
//   * Each wavefront owns 32 query rows.  Its Q fragment stays in VGPRs for the whole pass
//     as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, or
//     v_mfma_i32_32x32x32_i8 on the int8 codes).
//   * Computing S^T instead of S puts one query per lane (lane % 32) in the MFMA result, so
//     a row's maximum and sum are in-lane reductions plus one exchange with lane ^ 32, and the
//     per-row rescale of the output is a per-lane scalar.
//   * The P^T tile left in the accumulator registers is directly the B operand of
//     O^T += V^T P^T (bf16 MFMA): no LDS round trip for P.  Its key order inside each
//     16-key step is a fixed permutation, which V^T in LDS is stored in.
//   * K tiles (64 keys) are staged row-major and V tiles transposed (V^T, channel-major) in
//     LDS, double-buffered: global loads of tile t+1 are in flight while tile t computes.
//     16-byte LDS chunks are XOR-swizzled so every 16-lane phase of a ds_read_b128 hits 16
//     distinct bank groups.
//   * Workgroup ids are remapped so the workgroups the dispatcher places on one XCD (ids
//     congruent mod 8) process consecutive query tiles of the same head and share its K/V
//     stream in that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace ditattn {

namespace {

constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kBQ = 128;        // query rows per workgroup (= int8 Q block)
constexpr int kBK = 64;         // keys per tile (= int8 K block)
constexpr float kLog2e = 1.4426950408889634f;

template <int D, bool INT8>
struct Tile {
  static constexpr int KROW = INT8 ? D : 2 * D;  // bytes per K row
  static constexpr int KCH = KROW / 16;          // 16-byte chunks per K row
  static constexpr int KRPG = 16 / KCH;          // K rows per 256-byte bank period
  static constexpr int KBYTES = kBK * KROW;
  static constexpr int VROW = 2 * kBK;           // bytes per V^T row (one channel, 64 keys)
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int NKL = kBK * KCH / kThreads;  // 16-byte K loads per thread per tile
  static constexpr int KG = D / 32;                 // keys per thread in the V transpose
  static constexpr int VDC = D / 8;                 // 8-channel groups per V row
  static constexpr int NQF = INT8 ? D / 32 : D / 16;  // 16-byte Q fragments per lane
  static constexpr int NDB = D / 32;                // 32-channel output blocks
  static_assert(NKL >= 1 && KCH <= 16, "tile shape");
};

// Position of key k (0..63) in a V^T row: inside each 16-key step the keys are ordered
// {0-3, 8-11, 4-7, 12-15}, the order in which the S^T accumulator of lane half h holds them.
__device__ __forceinline__ int vpos(int k) {
  const int g = (k >> 2) & 3;
  return (k & ~15) | ((g & 1) << 3) | ((g >> 1) << 2) | (k & 3);
}

// Byte offset of 16-byte chunk `ch` of K row `key` in the swizzled K tile.
template <int D, bool INT8>
__device__ __forceinline__ int koff(int key, int ch) {
  using T = Tile<D, INT8>;
  return key * T::KROW + ((ch ^ ((key / T::KRPG) % T::KCH)) << 4);
}

// Byte offset of 16-byte chunk `ch` (0..7) of V^T row `d` in the swizzled V^T tile.
__device__ __forceinline__ int voff(int d, int ch) {
  return d * (2 * kBK) + ((ch ^ ((d >> 1) & 7)) << 4);
}

template <int D, bool INT8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_kernel(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ kp,
                     const uint8_t* __restrict__ vp, float* __restrict__ op,
                     const float* __restrict__ q_scale, const float* __restrict__ k_scale,
                     int S, int n_qt, float c) {
  using T = Tile<D, INT8>;
  constexpr int EB = INT8 ? 1 : 2;  // bytes per Q/K element
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // XCD-aware remap: the dispatcher sends workgroup i to XCD i % 8; give each XCD a
  // contiguous range of logical tiles.
  const int nwg = gridDim.x;
  const int wg = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = wg & 7;
  const int L = xcd * per + min(xcd, rem) + (wg >> 3);
  const int bh = L / n_qt;
  const int qt = L - bh * n_qt;

  const size_t head = (size_t)bh * (size_t)S * D;  // element offset of this (b, h)
  const uint8_t* kh = kp + head * EB;
  const uint8_t* vh = vp + head * 2;
  const int nkt = (S + kBK - 1) / kBK;

  // ---- Q fragment: B operand, lane holds query q, channels [32f + 16hh, +16) bytes ------
  const int q = qt * kBQ + wave * 32 + l32;
  u32x4 qf[T::NQF];
  {
    const uint8_t* qrow = qp + (head + (size_t)min(q, S - 1) * D) * EB;
#pragma unroll
    for (int f = 0; f < T::NQF; ++f) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qrow + f * 32 + hh * 16);
      qf[f] = (q < S) ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float cq = c;
  if constexpr (INT8) cq = q_scale[(size_t)bh * n_qt + qt] * c;

  // ---- staging of one K/V tile: global -> registers -> LDS -------------------------------
  u32x4 kreg[T::NKL];
  u32x4 vreg[T::KG];
  const int vdc = tid % T::VDC;   // this thread's 8-channel group of V
  const int vkg = tid / T::VDC;   // this thread's group of KG keys

  auto gload = [&](int kt) {
    const int key0 = kt * kBK;
#pragma unroll
    for (int r = 0; r < T::NKL; ++r) {
      const int id = tid + r * kThreads;
      const int key = id / T::KCH, ch = id % T::KCH;
      const int row = key0 + key;
      kreg[r] = (row < S) ? *reinterpret_cast<const u32x4*>(kh + (size_t)row * T::KROW + ch * 16)
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < T::KG; ++i) {
      const int row = key0 + vkg * T::KG + i;
      vreg[i] = (row < S) ? *reinterpret_cast<const u32x4*>(vh + ((size_t)row * D + vdc * 8) * 2)
                          : u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto lstore = [&](int buf) {
    uint8_t* sk = smem + buf * T::BUF;
    uint8_t* sv = sk + T::KBYTES;
#pragma unroll
    for (int r = 0; r < T::NKL; ++r) {
      const int id = tid + r * kThreads;
      const int key = id / T::KCH, ch = id % T::KCH;
      *reinterpret_cast<u32x4*>(sk + koff<D, INT8>(key, ch)) = kreg[r];
    }
    // transpose KG keys x 8 channels into 8 channel rows of KG consecutive positions
    const int pos = vpos(vkg * T::KG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = vdc * 8 + e;
      uint32_t w[T::KG];
#pragma unroll
      for (int i = 0; i < T::KG; ++i) w[i] = (e & 1) ? (vreg[i][e >> 1] >> 16) : (vreg[i][e >> 1] & 0xFFFFu);
      const int off = voff(d, pos >> 3) + ((pos & 7) << 1);
      if constexpr (T::KG == 4) {
        *reinterpret_cast<u32x2*>(sv + off) = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
      } else {
        *reinterpret_cast<uint32_t*>(sv + off) = w[0] | (w[1] << 16);
      }
    }
  };

  f32x16 oacc[T::NDB];
#pragma unroll
  for (int db = 0; db < T::NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // running max of the scaled (log2-domain) scores of row q
  float l_run = 0.f;        // this lane's share of the running row sum

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* sk = smem + buf * T::BUF;
    const uint8_t* sv = sk + T::KBYTES;

    // ---- S^T = K Q^T: lane holds keys 32kb + 8j + 4hh + i (register 4j + i), query q ----
    float s[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kb * 32 + l32;
      if constexpr (INT8) {
        i32x16 acc = i32x16{};
#pragma unroll
        for (int f = 0; f < T::NQF; ++f) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(sk + koff<D, INT8>(key, 2 * f + hh));
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                      __builtin_bit_cast(i32x4, qf[f]), acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (float)acc[r];
      } else {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int f = 0; f < T::NQF; ++f) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(sk + koff<D, INT8>(key, 2 * f + hh));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, qf[f]), acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = acc[r];
      }
    }

    // keys past the end of the sequence get zero weight
    if (kt == nkt - 1 && (S % kBK) != 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kBK + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key >= S) s[kb][r] = -INFINITY;
        }
    }

    // ---- online softmax in the log2 domain: t = s * cf, p = 2^(t - m) ----------------
    float cf = cq;
    if constexpr (INT8) cf = cq * k_scale[(size_t)bh * nkt + kt];
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xor32_max(mx);
    const float m_new = fmaxf(m_run, mx * cf);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[c4 >> 1][8 * (c4 & 1) + e], cf, -m_new));
        psum += p;
        pb[c4][e] = (__bf16)p;
      }
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T P^T: lane holds channels 32db + 8j + 4hh + i, query q -------------
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      const int d = db * 32 + l32;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(sv + voff(d, 2 * c4 + hh));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[c4],
                                                           oacc[db], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, fp32 -------------------------------------------------------
  const float inv = 1.f / xor32_sum(l_run);
  if (q < S) {
    float* orow = op + head + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 o4 = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv, oacc[db][4 * j + 2] * inv,
                    oacc[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * j + 4 * hh) = o4;
      }
  }
}

template <int D, bool INT8>
hipError_t launch(const void* q, const void* k, const void* v, float* o, const float* qs,
                  const float* ks, int B, int H, int S, float scale, hipStream_t stream) {
  const int n_qt = (S + kBQ - 1) / kBQ;
  const long long nwg = (long long)B * H * n_qt;
  hipLaunchKernelGGL((attn_fwd_kernel<D, INT8>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(v), o, qs, ks, S, n_qt, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* q, const void* k, const void* v, float* o, int B, int H,
                            int S, int D, float scale, hipStream_t stream) {
  if (D == 64) return launch<64, false>(q, k, v, o, nullptr, nullptr, B, H, S, scale, stream);
  return launch<128, false>(q, k, v, o, nullptr, nullptr, B, H, S, scale, stream);
}

hipError_t launch_attn_int8(const void* q_codes, const void* k_codes, const void* v, float* o,
                            const float* q_scale, const float* k_scale, int B, int H, int S,
                            int D, float scale, hipStream_t stream) {
  if (D == 64)
    return launch<64, true>(q_codes, k_codes, v, o, q_scale, k_scale, B, H, S, scale, stream);
  return launch<128, true>(q_codes, k_codes, v, o, q_scale, k_scale, B, H, S, scale, stream);
}

}  // namespace ditattn
