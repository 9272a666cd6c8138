// Non-causal multi-head attention forward for gfx950 (MI355X): bf16, int8-QK and fp8-QK
// variants, and fp8 for both products.
//
// O = softmax(Q K^T * scale) V, computed blockwise on chip so the S x S score matrix never
// reaches HBM (the IO-aware tiling of the "Flash Attention 2 for Z-Image S3-DiT" page, method
// paragraph), with a streaming (online) softmax: a running row maximum m and row sum l; the
// output is rescaled by 2^(m_old - m_new) when m moves, and the final division by l makes the
// result exact attention up to rounding.
//
// Work decomposition (one workgroup = 8 wavefronts = 256 query rows of one (b, h); one
// workgroup per CU, i.e. two wavefronts per SIMD):
//   * Each wavefront owns 32 query rows.  Its Q fragment stays in VGPRs for the whole pass
//     as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16, v_mfma_i32_32x32x32_i8 on
//     int8 codes, or v_mfma_f32_32x32x64_f8f6f4 on fp8 e4m3 codes).  Computing S^T puts one query per lane (lane % 32) in the result,
//     so a row's maximum and sum are in-lane reductions plus one exchange with lane ^ 32
//     (v_permlane32_swap), and rescaling a row of the output is a per-lane scalar.
//   * The P^T tile left in the accumulator registers is directly the B operand of
//     O^T += V^T P^T (bf16 MFMA), no LDS round trip for P.  Inside each 16-key step its key
//     order is a fixed permutation, and the V^T A operand is read from LDS in that order
//     with ds_read_b64_tr_b16 (gfx950's transposing LDS read), so V stays row-major in LDS.
//     With fp8 V the weights are packed to e4m3 bytes and PV is one
//     v_mfma_f32_32x32x64_f8f6f4 per 32 channels, its V^T operand read with ds_read_b64_tr_b8;
//     each lane's sum of its rounded weights is one 16x16x128 fp8 product.
//   * K and V tiles of 64 keys go straight from global memory into LDS with
//     buffer_load_dwordx4 ... lds (no VGPR staging).  Each wave writes 1 KB contiguously per
//     instruction, so the XOR swizzle of 16-byte chunks is applied to the *global* address a
//     lane fetches: LDS slot p holds the chunk that belongs at p in the swizzled layout.  The
//     swizzles make every 16- and 32-lane phase of the MFMA operand reads conflict-free.
//   * Software pipeline, three independent streams per stage in one basic block: stage j
//     computes S[j+2] = K[j+2] Q^T on the matrix cores, turns S[j+1] into the weights P[j+1]
//     on the VALU, and accumulates O += V[j]^T P[j]; it issues the loads of K[j+3] and V[j+1]
//     (K runs three tiles ahead of V); one barrier per stage.  For bf16 at D = 128 the stage
//     asks the compiler for its exponential / matrix-product interleave, which spreads the
//     32 exponentials evenly between the 32 products.
//   * Long calls with bf16 V (and a workspace) first copy V into V^T tiles, each 16-key step in
//     the order the P^T operand holds its keys, so a PV operand is one 16-byte LDS read.
//   * int8 scores leave the matrix cores already as fp32: the integer accumulator starts at
//     the bit pattern of 1.5 * 2^23, so its final bits read as fp32 are 1.5 * 2^23 plus the
//     score, exactly; the bias folds into the exponent offset (no conversion instructions).
//   * Lazy, optimistic rescale: the weights of a tile are formed with the current offset m
//     straight away; only when one would exceed 2^8 (seen through each lane's sum of its
//     weights, which bounds them all) does the tile take its row maximum, move m, rescale O
//     and redo the weights.  Weights up to 2^8 are used as they are (bf16 and fp32 hold them
//     with full relative precision); on typical data m moves a handful of times per row, so
//     the row maximum is almost never computed.
//   * Workgroup ids are remapped so the workgroups the dispatcher places on one XCD (ids
//     congruent mod 8) process consecutive query tiles of the same head and share its K/V
//     stream in that XCD's L2.
//   * When the query tiles leave the last round of workgroups mostly empty (the call passes a
//     workspace), that round's tiles are cut along the key axis into one equal range per CU
//     and run by a second launch (split_plan.h); each part of a tile leaves its unnormalised
//     O, offset m and sum l in the workspace, and the last part to arrive merges them in key
//     order, so the output does not depend on timing.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "scale_index.h"
#include "split_plan.h"

namespace ditattn {

namespace {

// What Q and K hold, and V: bf16, int8 or fp8 codes for Q and K; bf16 V, or for kFp8All
// fp8 codes for V as well (PV on the fp8 matrix cores).
enum Kind { kBF16 = 0, kInt8 = 1, kFp8 = 2, kFp8All = 3 };

constexpr int kQBlock = 128;    // int8 / fp8 Q quantization block (tokens)
constexpr int kBK = 64;         // keys per tile (= int8 K block)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyW = 256.0f;  // 2^8: largest weight (and lane weight sum) kept as it is
// Calls with bf16 V over at least this many keys (D = 128, with a workspace) read V through V^T
// tiles written by a prepass: one 16-byte LDS read per PV operand instead of two transposing
// ones, 1.5-2% faster at S = 118800 (bf16, int8-QK, fp8-QK) with the prepass (a read and a
// write of V) included.  The prepass costs 2% of the bf16 call at S = 11440, as much as the
// tiles save there.
constexpr int kVtMinS = 32768;
// fp8 weights are formed 2^4 times larger (the small ones then fall in e4m3's normal range, not
// its coarse subnormals), and kept while their lane sum is <= 2^8, so every one is <= 256 < 448.
constexpr float kLog2WScale8 = 4.0f;
// 1.5 * 2^23: every fp32 in [2^23, 2^24) is an integer and consecutive integers have
// consecutive bit patterns, so bits(kBiasF) + n read as fp32 is kBiasF + n for |n| < 2^22.
// An int8 score is at most 127 * 127 * 128 < 2^21 in magnitude, so the int8 QK product
// accumulated onto bits(kBiasF) converts to fp32 without a conversion instruction.
constexpr float kBiasF = 12582912.0f;
// Word 3 of a raw buffer resource for gfx9-family parts: 32-bit data format, no swizzle, no
// index stride; the range check is against the byte count in word 2.
constexpr int kBufferFlags = 0x00020000;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

template <int D, bool INT8, int NW, bool V8 = false>
struct Tile {
  static constexpr int NT = 64 * NW;             // threads per workgroup
  static constexpr int BQ = 32 * NW;             // query rows per workgroup
  static constexpr int KROW = INT8 ? D : 2 * D;  // bytes per K row in LDS
  static constexpr int KCH = KROW / 16;          // 16-byte chunks per K row
  static constexpr int KRPG = 16 / KCH;          // K rows per 256-byte bank period
  static constexpr int KBYTES = kBK * KROW;      // one K tile
  static constexpr int VROW = V8 ? D : 2 * D;    // bytes per V row
  static constexpr int VCH = VROW / 16;
  static constexpr int VBYTES = kBK * VROW;      // one V tile
  static constexpr int KLD = (KBYTES / 16 + NT - 1) / NT;  // 16-byte loads per thread per K tile
  static constexpr int VLD = (VBYTES / 16 + NT - 1) / NT;
  static constexpr bool KPART = (KBYTES / 16) % NT != 0;  // last K load only on some threads
  static_assert((VBYTES / 16) % NT == 0 && (!KPART || KLD == 1), "tile shape");
  static constexpr int NQF = INT8 ? D / 32 : D / 16;   // 16-byte Q fragments per lane
  static constexpr int NDB = D / 32;                   // 32-channel output blocks
  static_assert(KCH <= 16, "tile shape");
  static_assert(kScaleQBlock == kQBlock && kScaleKBlock == kBK, "scale blocks");
};

// Swizzled chunk of K row `key`: 16 consecutive rows read at one logical chunk land in 16
// distinct bank groups.
template <int D, bool INT8>
__device__ __forceinline__ int kswz(int key, int ch) {
  using T = Tile<D, INT8, 4>;
  return ch ^ ((key / T::KRPG) % T::KCH);
}

// Swizzled chunk of V row `row`.  The transposing reads fetch 4 consecutive rows x 32 bytes per
// 16 lanes (two 16-lane groups side by side); XORing the chunk with a per-(row mod 4) mask
// spreads them over distinct bank groups for both 16- and 32-lane phases.
template <int D>
__device__ __forceinline__ int vswz(int row, int ch) {
  if constexpr (D == 128) {
    return ch ^ ((0xEA40 >> (4 * (row & 3))) & 0xF);  // masks {0, 4, 10, 14}
  } else {
    return ch ^ ((row & 2) << 1);  // masks {0, 0, 4, 4}
  }
}

// Swizzled chunk of fp8 V row `row` (128-byte rows, D = 128).  The transposing byte reads
// fetch 16 bytes of each of 8 rows per 16 lanes (rows 8 a + 4 h + 0..3, a = 0, 1, chunk pair
// of one 32-channel block); XORing the chunk with 2 bit1(row) + 4 bit3(row) spreads each 32-lane
// half over 16 distinct 16-byte bank groups.
__device__ __forceinline__ int vswz8(int row, int ch) {
  return ch ^ (2 * ((row >> 1) & 1) + 4 * ((row >> 3) & 1));
}

// An empty asm that the compiler must assume redefines x (a VGPR value).
__device__ __forceinline__ void opaque(uint32_t& x) { asm volatile("" : "+v"(x)); }

// N no-ops, executed once: they only move the code after them by 4 N bytes.
template <int N>
__device__ __forceinline__ void pad_nops() {
  if constexpr (N > 0) {
    asm volatile("s_nop 0");
    pad_nops<N - 1>();
  }
}

// Sizes and strides of one call (passed by value into the kernel's scalar argument segment).
// Strides are in elements of the respective tensor; the channel axis is contiguous.  The
// pointers stay separate __restrict__ arguments: only then may the per-tile K scale be read
// with a scalar load, which does not wait for the K/V tile copies in flight.
struct KArgs {
  int64_t qsb, qsh, qss, ksb, ksh, kss, vsb, vsh, vss, osb, osh, oss;
  int H;
  int Sq;                  // query rows per (b, h)
  int Sk;                  // keys per (b, h)
  int n_qt;                // query tiles per (b, h)
  float c;                 // scale * log2(e)
  int o_bf16;
  SplitPlan plan;          // whole tiles, and the last round shared out over the key axis
};

// q, k: bf16 Q and K, or the int8 codes; v: bf16 V; o: fp32 or bf16 O; lse: fp32 [B, H, Sq]
// natural-log normalisers, or null; q_scale / k_scale: the int8 path's per-block scales.
// TAIL false: one workgroup per whole tile, the first a.plan.n_main tiles (and, when cnt is
// not null, workgroup 0 zeroes the a.plan.n_tail arrival counters for the tail launch that
// follows).  TAIL true: a.plan.G workgroups share the a.plan.n_tail tiles after those (see
// split_plan.h); part / cnt: the slots of the parts of split tiles and one arrival counter
// per tail tile (zero at launch, left zero).  Two kernels, so that the whole-tile one, which
// does nearly all the work, is compiled without any of the tail's code.
// At D = 64 the wave count per SIMD is capped at two as well: one 8-wave workgroup per CU is
// the design and a third wave slot could not hold a second workgroup, yet aiming for three
// squeezes the kernel into 168 VGPRs and serialises its K fragment reads behind the products.
// (At D = 128 the cap changes nothing but the instruction schedule, measurably for the worse.)
// VT: vp holds the V^T tiles of vt_tiles_kernel (the kinds with bf16 V, D = 128) instead of V.
template <int D, int KIND, int NW, bool TAIL, bool VT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, D == 64 ? 2 : 8)))
void attn_fwd_kernel(const uint8_t* __restrict__ qp, const uint8_t* __restrict__ kp,
                     const uint8_t* __restrict__ vp, uint8_t* __restrict__ op,
                     float* __restrict__ lse, const float* __restrict__ q_scale,
                     const float* __restrict__ k_scale, const float* __restrict__ v_scale,
                     float* __restrict__ part, int* __restrict__ cnt, const KArgs a) {
  const int Sq = a.Sq, Sk = a.Sk, n_qt = a.n_qt;
  const float c = a.c;
  constexpr bool INT8 = KIND != kBF16;  // one-byte Q/K codes (int8 or fp8)
  constexpr bool I8 = KIND == kInt8;
  constexpr bool F8 = KIND == kFp8 || KIND == kFp8All;
  constexpr bool V8 = KIND == kFp8All;  // fp8 V codes, PV on the fp8 matrix cores
  static_assert(!V8 || D == 128, "fp8 V is laid out for D = 128");
  static_assert(!VT || (D == 128 && !V8), "V^T tiles: bf16 V, D = 128");
  using T = Tile<D, INT8, NW, V8>;
  constexpr int EBV = V8 ? 1 : 2;       // bytes per V element
  constexpr int kThreads = T::NT;
  constexpr int kBQ = T::BQ;
  constexpr int EB = INT8 ? 1 : 2;  // bytes per Q/K element
  // Four distinct LDS objects, so the compiler can tell the buffer being read from the one an
  // in-flight global->LDS load is filling and does not wait for that load early.
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf_0[T::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf_1[T::KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf_0[T::VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf_1[T::VBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int nkt = (Sk + kBK - 1) / kBK;
  __shared__ int s_last;  // the merge decision of a split tile, for the whole workgroup

  const SplitPlan plan = a.plan;
  const int wg = blockIdx.x;
  const int w_tail = TAIL ? xcd_order(wg, plan.G) : -1;  // tail workgroup index

  if constexpr (!TAIL) {
    if (cnt != nullptr && wg == 0)
      for (int i = tid; i < plan.n_tail; i += kThreads) cnt[i] = 0;
  }
  // One pass over query tile L (its rows of one (b, h)) and key tiles [kbeg, kend) per
  // iteration: the whole tile of this workgroup, or (TAIL) each of its segments, the one that
  // starts a tile first (see split_plan.h).  A whole tile writes O; a part of a split tile
  // (segment seg, on tail tile tt) goes through the merge.
  for (int it = 0; it < (TAIL ? 2 : 1); ++it) {
    int L, kbeg, kend, tt = 0, seg = 0;
    if constexpr (!TAIL) {
      L = xcd_order(wg, plan.n_main);
      kbeg = 0;
      kend = nkt;
    } else {
      seg = 1 - it;
      if (!tail_segment(plan, w_tail, seg, tt, kbeg, kend)) continue;
      // (uniform values: kept in scalar registers, whatever unit the divisions ran on)
      tt = __builtin_amdgcn_readfirstlane(tt);
      kbeg = __builtin_amdgcn_readfirstlane(kbeg);
      kend = __builtin_amdgcn_readfirstlane(kend);
      L = plan.n_main + tt;
    }
    const int bh = L / n_qt;
    const int qt = L - bh * n_qt;

    const int bb = bh / a.H, hd = bh - bb * a.H;
    const uint8_t* kh = kp + (bb * a.ksb + hd * a.ksh) * EB;   // first key row of this (b, h)
    // (V^T tiles: nkt contiguous tiles per (b, h))
    const uint8_t* vh = VT ? vp + (size_t)bh * nkt * T::VBYTES : vp + (bb * a.vsb + hd * a.vsh) * EBV;
    const int64_t krs = a.kss * EB, vrs = a.vss * EBV;          // bytes between key / value rows

    // ---- Q fragment: B operand; lane holds query q, bytes [32f + 16hh, +16) of its row -------
    const int q = qt * kBQ + wave * 32 + l32;
    u32x4 qf[T::NQF];
    {
      const uint8_t* qrow = qp + (bb * a.qsb + hd * a.qsh + (int64_t)min(q, Sq - 1) * a.qss) * EB;
#pragma unroll
      for (int f = 0; f < T::NQF; ++f) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + f * 32 + hh * 16);
        qf[f] = (q < Sq) ? x : u32x4{0u, 0u, 0u, 0u};
      }
    }
    // fp8 V: the A operand of the weight-sum product.  In a 16x16x128 fp8 product the bytes of
    // lane l are row l % 16 of A, or column l % 16 of B, over the same k group l / 16, and lane l
    // receives result rows 4 (l / 16) .. +3 of column l % 16.  Row m takes k group m / 4 alone
    // (e4m3 1.0, 0x38, where l / 16 == (l % 16) / 4, else 0), so result (m, n) is the byte sum
    // of B lane 16 (m / 4) + n: for every lane, its own bytes.
    i32x8 rsel = {};
    if constexpr (V8) {
      const int one = ((lane >> 4) & 3) == ((lane >> 2) & 3) ? 0x38383838 : 0;
      rsel = i32x8{one, one, one, one, one, one, one, one};
    }
    float cq = c;
    if constexpr (INT8) {
      const int nqb = (Sq + kQBlock - 1) / kQBlock;  // (the int8 path never samples: Sq = Sk)
      cq = q_scale[(size_t)bh * nqb + q_scale_block(qt, wave, kBQ, nqb)] * c;
    }

    // ---- direct global -> LDS tile loads ------------------------------------------------
    // Slot p (16 bytes) of a tile is written by lane p % 64 of wave (p / 64) % NW in
    // instruction p / (64 NW) (an int8 D = 64 K tile has fewer slots than threads: the waves
    // past its end skip it).  The byte offset each lane fetches from, relative to the tile's
    // first row, is loop invariant (one VGPR per instruction) and the tile base is
    // wave-uniform (the base of the buffer resource, in SGPRs), so a load needs no vector
    // address arithmetic.  Every tile is a full 64 rows: a partial last tile is read as the last 64
    // rows of the sequence instead (keys it shares with the previous tile are masked to -inf,
    // so they get weight 0), and only a sequence shorter than one tile clamps its rows to the
    // last one.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t kofl[T::KLD], vofl[T::VLD];
#pragma unroll
    for (int r = 0; r < T::KLD; ++r) {
      const int p = r * kThreads + tid;
      const int key = p / T::KCH, pch = p % T::KCH;
      kofl[r] = (uint32_t)(key * krs) + kswz<D, INT8>(key, pch) * 16;
    }
#pragma unroll
    for (int r = 0; r < T::VLD; ++r) {
      const int p = r * kThreads + tid;
      if constexpr (VT) {
        // a V^T tile: 128 channel rows of 64 keys (128 bytes), swizzled as an int8 K tile
        const int row = p / 8, pch = p % 8;
        vofl[r] = (uint32_t)(row * 128) + kswz<128, true>(row, pch) * 16;
      } else {
        const int key = p / T::VCH, pch = p % T::VCH;
        vofl[r] = (uint32_t)(key * vrs) + (V8 ? vswz8(key, pch) : vswz<D>(key, pch)) * 16;
      }
    }
    // The tile copies are buffer loads with the LDS as destination (MUBUF), on a buffer resource
    // whose base is the tile's first row and whose range covers every 32-bit offset.  The
    // compiler counts these as vector-memory operations only; the global (FLAT) form of the same
    // copy makes it treat each one as touching both memory and LDS, so while one is in flight
    // every LDS read has to drain the whole LDS queue (lgkmcnt(0)) instead of waiting for its own
    // result.  Measured: 7-10% faster at S = 4608 and 3% at S = 11440, unchanged at S = 118800.
    auto tile_dma = [&](const uint8_t* tb, uint32_t off, uint8_t* dst) __attribute__((always_inline)) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tb), 0, -1, kBufferFlags),
          (lds_void*)dst, 16, off, 0, 0, 0);
    };
    // First row of tile kt: kt * kBK, except a ragged last tile, which starts at Sk - kBK
    // (Sk >= kBK whenever more than one tile exists).  Tiles of K and of V are each loaded once,
    // in order from kbeg, so their base addresses advance by one tile per load (uniform, in SGPRs).
    const int64_t k_step = kBK * krs, v_step = VT ? (int64_t)T::VBYTES : kBK * vrs;
    const uint8_t* k_next = kh + kbeg * k_step;
    const uint8_t* v_next = vh + kbeg * v_step;
    const uint8_t* const k_last = kh + (int64_t)max(Sk - kBK, 0) * krs;
    const uint8_t* const v_last =
        VT ? vh + (int64_t)(nkt - 1) * T::VBYTES : vh + (int64_t)max(Sk - kBK, 0) * vrs;
    // The offsets are redefined (by an empty asm) at the top of every loop iteration, so their
    // zero extension cannot be hoisted out of the loop and each address is selected as scalar
    // base + 32-bit vector offset (the global "saddr" form), not a 64-bit VALU add.
    auto load_k = [&](int kt, uint8_t* dst) {
      const uint8_t* tb = kt == nkt - 1 ? k_last : k_next;
      k_next += k_step;
      if (T::KPART && wave_u * 64 >= T::KBYTES / 16) return;  // this wave has no K slot
#pragma unroll
      for (int r = 0; r < T::KLD; ++r) {
        const uint32_t off = kofl[r];  // (a subscript inside the builtin's argument drops the
                                       // kernel's host launch stub with this compiler)
        tile_dma(tb, off, dst + (r * kThreads + wave_u * 64) * 16);
      }
    };
    auto load_v = [&](int kt, uint8_t* dst) {
      const uint8_t* tb = kt == nkt - 1 ? v_last : v_next;
      v_next += v_step;
#pragma unroll
      for (int r = 0; r < T::VLD; ++r) {
        const uint32_t off = vofl[r];
        tile_dma(tb, off, dst + (r * kThreads + wave_u * 64) * 16);
      }
    };
    // the single tile of a sequence shorter than kBK: rows clamped to Sk - 1 (buffer loads as
    // the others: no global (FLAT) form anywhere, so the compiler never has to assume that an
    // LDS wait might also cover one and drain the whole LDS queue instead)
    auto load_short = [&](uint8_t* kdst, uint8_t* vdst) {
#pragma unroll
      for (int r = 0; r < T::KLD; ++r) {
        if (T::KPART && wave_u * 64 >= T::KBYTES / 16) break;
        const int p = r * kThreads + tid;
        const int key = p / T::KCH, pch = p % T::KCH;
        const uint32_t off = (uint32_t)(min(key, Sk - 1) * krs) + kswz<D, INT8>(key, pch) * 16;
        tile_dma(kh, off, kdst + (r * kThreads + wave_u * 64) * 16);
      }
#pragma unroll
      for (int r = 0; r < T::VLD; ++r) {
        const int p = r * kThreads + tid;
        const int key = p / T::VCH, pch = p % T::VCH;
        const uint32_t off =
            VT ? vofl[r]  // a V^T tile is always whole (its rows past Sk are zeros)
               : (uint32_t)(min(key, Sk - 1) * vrs) + (V8 ? vswz8(key, pch) : vswz<D>(key, pch)) * 16;
        tile_dma(vh, off, vdst + (r * kThreads + wave_u * 64) * 16);
      }
    };

    // ---- per-lane LDS read offsets (loop invariant) --------------------------------------
    // K (A operand of S^T = K Q^T): lane reads row kb2 * 32 + l32, logical chunk 2f + hh.
    int koffs[T::NQF];
#pragma unroll
    for (int f = 0; f < T::NQF; ++f) koffs[f] = l32 * T::KROW + kswz<D, INT8>(l32, 2 * f + hh) * 16;
    // V (A operand of O^T = V^T P^T) via ds_read_b64_tr_b16: 16-lane group g = lane / 16 covers
    // channels n0 = 32 db + 16 (g % 2) .. +15 and keys 16 c4 + 8 part + 4 hh + 0..3; lane j of
    // the group addresses row (j / 4) of those four and channels n0 + 4 (j % 4) .. +3.
    const int gj = lane & 15;
    const int vrow = 4 * hh + (gj >> 2);
    int voffs[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) {
      if constexpr (V8) {
        // fp8 V via ds_read_b64_tr_b8: in each 16-lane group lane t receives byte t % 8 of the
        // 8-byte rows addressed by lanes 2 m + t / 8 (m = 0..7).  Lanes 2m and 2m + 1 address
        // key k_m at channels n0 .. n0 + 7 and n0 + 8 .. n0 + 15, so lane t gets channel n0 + t
        // for the keys k_0..k_7: with n0 = 32 db + 16 (g % 2) and k_m = 16 i + 8 (m / 4) + 4 hh
        // + m % 4 for read i = 0..3, the lane's 32 bytes are its channel's values at exactly the
        // keys (and in the order) its 32 weights occupy in the P^T operand.
        const int m = gj >> 1;
        const int r0 = 8 * (m >> 2) + 4 * hh + (m & 3);
        const int f = 2 * ((r0 >> 1) & 1) + 4 * ((r0 >> 3) & 1);
        voffs[db] = r0 * T::VROW + (((2 * db) ^ f) + ((lane >> 4) & 1)) * 16 + 8 * (gj & 1);
      } else {
        const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (gj & 3);
        voffs[db] = vrow * T::VROW + vswz<D>(vrow, col >> 3) * 16 + (col & 7) * 2;
      }
    }

    // V^T (VT): lane reads channel row 32 db + l32, logical chunk 2 c4 + hh (the 8 keys of its
    // half of 16-key step c4, stored in P^T order); the swizzle does not depend on db.
    int vtoffs[VT ? 4 : 1];
    if constexpr (VT) {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) vtoffs[c4] = l32 * 128 + kswz<128, true>(l32, 2 * c4 + hh) * 16;
    }

    f32x16 oacc[T::NDB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // offset of row q's weights: a past maximum of its scaled scores
    float l_run = 0.f;        // this lane's share of the running row sum

    i32x16 ibias;
#pragma unroll
    for (int r = 0; r < 16; ++r) ibias[r] = (int)__builtin_bit_cast(uint32_t, kBiasF);
    if constexpr (I8) asm volatile("" : "+v"(ibias));  // an opaque VGPR tuple, not a splat

    // S^T tile of one K buffer: register 16 kb2 + r of lane holds key 32 kb2 + 8 (r / 4) +
    // 4 hh + r % 4, query q.  The int8 variant holds kBiasF + the integer score.
    auto qk = [&](const uint8_t* kbuf, float (&s)[32]) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        if constexpr (F8) {
          // fp8 e4m3 codes, 64 of each row per product: a lane's two 16-byte fragments f and
          // f + 1 (bytes [32f + 16hh, +16) and [32f + 32 + 16hh, +16) of its row) form one
          // operand.  Which k a byte stands for does not matter as long as both operands use
          // the same layout, and they do: both are the rows' own bytes at the same offsets.
          f32x16 acc = f32x16{};
#pragma unroll
          for (int f = 0; f < T::NQF; f += 2) {
            const u32x4 a0 = *reinterpret_cast<const u32x4*>(kbuf + kb2 * 32 * T::KROW + koffs[f]);
            const u32x4 a1 = *reinterpret_cast<const u32x4*>(kbuf + kb2 * 32 * T::KROW + koffs[f + 1]);
            const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                             (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
            const i32x8 b = {(int)qf[f][0], (int)qf[f][1], (int)qf[f][2], (int)qf[f][3],
                             (int)qf[f + 1][0], (int)qf[f + 1][1], (int)qf[f + 1][2], (int)qf[f + 1][3]};
            // formats 0, 0: both operands e4m3; no block scales (the scales are applied with
            // the softmax's exponent FMA)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s[16 * kb2 + r] = acc[r];
        } else if constexpr (I8) {
          // The accumulator starts at the bit pattern of kBiasF, so it ends as kBiasF + the
          // integer dot product, which read as fp32 is exactly that sum (see kBiasF)
          i32x16 acc;
#pragma unroll
          for (int f = 0; f < T::NQF; ++f) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(kbuf + kb2 * 32 * T::KROW + koffs[f]);
            if (f == 0) {
              // first product reads the bias tuple as C and writes a separate accumulator (the
              // builtin would copy the tuple first); s_nop 1 covers a VALU-written operand
              asm volatile("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, %3"
                           : "=&v"(acc) : "v"(a), "v"(qf[f]), "v"(ibias));
            } else {
              acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                          __builtin_bit_cast(i32x4, qf[f]), acc, 0, 0, 0);
            }
          }
          // (bit-cast the whole vector: a bit_cast of one subscripted element is miscompiled
          // to element 0 by this compiler)
          const f32x16 accf = __builtin_bit_cast(f32x16, acc);
#pragma unroll
          for (int r = 0; r < 16; ++r) s[16 * kb2 + r] = accf[r];
        } else {
          f32x16 acc = f32x16{};
#pragma unroll
          for (int f = 0; f < T::NQF; ++f) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(kbuf + kb2 * 32 * T::KROW + koffs[f]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qf[f]), acc, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s[16 * kb2 + r] = acc[r];
        }
      }
    };

    // Masks the keys tile jt does not own (a partial last tile: keys outside [jt * kBK, Sk) were
    // already seen in tile jt - 1, or lie past the end).  In tile-local key numbers the valid
    // range is [lo, hi); the empty asm keeps the comparisons inside the rarely taken branch.
    auto mask_tile = [&](int jt, float (&s)[32]) __attribute__((always_inline)) {
      if (jt == nkt - 1 && (Sk % kBK) != 0) {
        const int t0 = max(Sk - kBK, 0);  // the tile's first row
        int lo = jt * kBK - t0 - 4 * hh, hi = Sk - t0 - 4 * hh;
        asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int r = 0; r < 32; ++r) {
          const int kc = 32 * (r >> 4) + 8 * ((r >> 2) & 3) + (r & 3);
          if (kc < lo || kc >= hi) s[r] = -INFINITY;
        }
      }
    };

    // P of tile jt from its scores, optimistically with the current offset m_run: the tile's
    // row maximum is only needed when some weight would exceed kLazyW, and this lane's sum of
    // its 32 bf16 weights (lt) bounds every one of them.
    auto weights = [&](int jt, const float (&s)[32], bf16x8 (&pb)[4], float& lt, float& cf)
                       __attribute__((always_inline)) {
      cf = cq;
      if constexpr (INT8) cf = cq * k_scale[(size_t)bh * nkt + k_scale_block(jt, nkt)];
      // exponent offset: m_run, plus the bias carried by the int8 scores (cf * kBiasF, rounded
      // once; its error is far below the int8 quantization error of the scores themselves)
      const float mb = I8 ? fmaf(cf, kBiasF, m_run) : m_run;
      if constexpr (V8) {
        // fp8 weights (2^4 times the softmax weights, see kLog2WScale8), four to a dword in the
        // order of s (the P^T operand's byte order), in pb[0] and pb[1]
        float w[32];
#pragma unroll
        for (int e = 0; e < 32; ++e)
          w[e] = __builtin_amdgcn_exp2f(fmaf(s[e], cf, kLog2WScale8 - mb));
        u32x4 pw[2];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          // (both halves of the word are written: the first conversion's "old" word is any
          // register, here its own source, so that no zero has to be materialised)
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(w[4 * d], w[4 * d + 1], __float_as_int(w[4 * d]), false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(w[4 * d + 2], w[4 * d + 3], word, true);
          pw[d >> 2][d & 3] = (uint32_t)word;
        }
        pb[0] = __builtin_bit_cast(bf16x8, pw[0]);
        pb[1] = __builtin_bit_cast(bf16x8, pw[1]);
        // This lane's sum of its 32 fp8 weights as they enter PV, on the matrix cores: the
        // packed weights are the B operand of a 16x16x128 product whose A (rsel) gives output
        // row m the k group m / 4 alone, so each output of lane l adds the 32 bytes of lane l
        // itself, exactly (at most 2^8 per weight: far inside fp32).
        const i32x8 pf = {(int)pw[0][0], (int)pw[0][1], (int)pw[0][2], (int)pw[0][3],
                          (int)pw[1][0], (int)pw[1][1], (int)pw[1][2], (int)pw[1][3]};
        const f32x4 rs = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            rsel, pf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        lt = rs[0];
      } else {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pb[c4][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 * c4 + e], cf, -mb));
        // row sum of the bf16 weights that enter PV, two at a time on the dot unit
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        lt = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            lt = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[c4][e], pb[c4][e + 1]}, ones, lt, false);
      }
    };

    // The rare path: a lane's weight sum above kLazyW (or inf / NaN, e.g. on the first tile)
    // makes the wave take the tile's row maximum, move m_run, rescale O and l (which then hold
    // the tiles before jt) and recompute the weights of tile jt.
    auto settle = [&](int jt, const float (&s)[32], bf16x8 (&pb)[4], float& lt)
                      __attribute__((always_inline)) {
      float cf;
      if (__builtin_amdgcn_ballot_w64(!(lt <= kLazyW)) != 0) {  // (V8: the sum of 2^4 w <= 2^8)
        cf = cq;
        if constexpr (INT8) cf = cq * k_scale[(size_t)bh * nkt + jt];
        float mx;
        if constexpr (I8) {
          // biased int8 scores are positive floats (or -inf when masked): their bit patterns
          // order like signed integers
          int mi = __float_as_int(s[0]);
#pragma unroll
          for (int r = 1; r < 32; ++r) mi = max(mi, __float_as_int(s[r]));
          mx = __int_as_float(xor32_max_i32(mi)) - kBiasF;  // exact: integers below 2^24
        } else {
          mx = s[0];
#pragma unroll
          for (int r = 1; r < 32; ++r) mx = fmaxf(mx, s[r]);
          mx = xor32_max(mx);
        }
        const float m_new = fmaxf(m_run, mx * cf);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) oacc[db] *= alpha;
        weights(jt, s, pb, lt, cf);
      }
      l_run += lt;
    };

    // One pipeline stage j: S[j+2] = K[j+2] Q^T on the matrix cores, the weights P[j+1] of
    // S[j+1] on the VALU, and O += V[j]^T P[j] — three independent streams in one basic block —
    // then the rare rescale for tile j + 1, which must follow the PV products of tile j.
    auto stage = [&](int j, auto par_c, float (&s1)[32], float (&s2)[32], bf16x8 (&p0)[4],
                     bf16x8 (&p1)[4]) __attribute__((always_inline)) {
      constexpr int par = decltype(par_c)::value;
      uint8_t* const kb_read = par ? kbuf_1 : kbuf_0;   // holds K[j+2]
      uint8_t* const kb_fill = par ? kbuf_0 : kbuf_1;   // held K[j+1]; receives K[j+3]
      uint8_t* const vb_cur = par ? vbuf_1 : vbuf_0;    // holds V[j]
      uint8_t* const vb_next = par ? vbuf_0 : vbuf_1;   // receives V[j+1]
      if (j + 3 < kend) load_k(j + 3, kb_fill);
      if (j + 1 < kend) load_v(j + 1, vb_next);

      // bf16 at D = 128: the compiler's interleave of exponentials with matrix products for
      // this block (2-3% faster; the 8-bit kinds and D = 64 run slower with it).  8-bit QK on
      // V^T tiles: its interleave of LDS reads with products (with the tiles 1.5-1.9% faster on
      // int8-QK and 1.6% on fp8-QK than reading V as it is; on int8-QK it loses without them).
      if constexpr (KIND == kBF16 && D == 128) __builtin_amdgcn_iglp_opt(3);
      if constexpr ((KIND == kInt8 || KIND == kFp8) && D == 128 && VT) __builtin_amdgcn_iglp_opt(0);
      // (past the last tile these compute on stale data and are discarded)
      qk(kb_read, s2);
      float lt, cf;
      weights(j + 1, s1, p1, lt, cf);

      // O^T += V[j]^T P[j]: lane holds channels 32 db + 8 (r / 4) + 4 hh + r % 4, query q
      if constexpr (V8) {
        const u32x4 pw0 = __builtin_bit_cast(u32x4, p0[0]), pw1 = __builtin_bit_cast(u32x4, p0[1]);
        const i32x8 pf = {(int)pw0[0], (int)pw0[1], (int)pw0[2], (int)pw0[3],
                          (int)pw1[0], (int)pw1[1], (int)pw1[2], (int)pw1[3]};
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          const uint8_t* base = vb_cur + voffs[db];
          i32x8 va;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // keys 16 i + ...: 16 rows further on per read
            const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 16 * i * T::VROW));
            va[2 * i] = x[0];
            va[2 * i + 1] = x[1];
          }
          oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pf, oacc[db], 0, 0, 0, 0, 0, 0);
        }
      } else {
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          u32x4 a;
          if constexpr (VT) {
            a = *reinterpret_cast<const u32x4*>(vb_cur + vtoffs[c4] + db * 32 * 128);
          } else {
            const uint8_t* base = vb_cur + voffs[db] + 16 * c4 * T::VROW;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * T::VROW));
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            a = u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
          }
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), p0[c4],
                                                             oacc[db], 0, 0, 0);
        }
      }
      }
      if (j + 1 < kend) settle(j + 1, s1, p1, lt);
      mask_tile(j + 2, s2);
      // the loads into kb_fill / vb_next must land before any wave reads them
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
    };

    // ---- prologue (tiles counted from kbeg): S[0], S[1] and P[0] computed; K[2] and V[0]
    // resident.  A sequence shorter than one tile is never split (kbeg = 0, kend = 1).
    if (Sk < kBK) {
      load_short(kbuf_0, vbuf_0);
    } else {
      load_k(kbeg, kbuf_0);
      if (kbeg + 1 < kend) load_k(kbeg + 1, kbuf_1);
      load_v(kbeg, vbuf_0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    float sa[32], sb[32];
    bf16x8 pa[4], pbb[4];
    qk(kbuf_0, sa);
    if (kbeg + 1 < kend) qk(kbuf_1, sb);
    __syncthreads();  // every wave has read K[0] and K[1]
    if (kbeg + 2 < kend) load_k(kbeg + 2, kbuf_0);
    mask_tile(kbeg, sa);
    if (kbeg + 1 < kend) mask_tile(kbeg + 1, sb);
    {
      float lt, cf;
      weights(kbeg, sa, pa, lt, cf);
      settle(kbeg, sa, pa, lt);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    // Where the main loop lands in the instruction stream matters: shifting the same loop by
    // 4-byte steps moved the long-video int8 call by up to 3% (shifts that are a multiple of 8
    // bytes from the unpadded placement were the slow ones) and the bf16 call by up to 1%.
    // These pads are the measured best for this loop and compiler.
    pad_nops<KIND == kInt8 ? (VT ? 3 : 2) : VT ? 0 : 3>();

    // stage j reads S[j+1] and writes S[j+2]; consumes P[j] and produces P[j+1]
    int j = kbeg;
    for (; j + 1 < kend; j += 2) {
#pragma unroll
      for (int r = 0; r < T::KLD; ++r) opaque(kofl[r]);
#pragma unroll
      for (int r = 0; r < T::VLD; ++r) opaque(vofl[r]);
      stage(j, std::integral_constant<int, 0>{}, sb, sa, pa, pbb);
      stage(j + 1, std::integral_constant<int, 1>{}, sa, sb, pbb, pa);
    }
    if (j < kend) stage(j, std::integral_constant<int, 0>{}, sb, sa, pa, pbb);

    // ---- a part of a split tile: leave the partial result; the last to arrive merges -------
    // Partial of a part (slot of its workgroup and segment): each lane's O accumulator, then
    // each lane's (m, l); lane-major per 16-byte column so every store and load of a wave is
    // 1 KB contiguous.  The part that arrives last merges every part in key order, the others
    // from their slots and its own from registers: the result is the same whichever part that
    // is.  It is nearly always the part holding the tile's first keys (the second segment of
    // its workgroup, which ends last), and that part finds the others already arrived before
    // leaving its own: it skips its store.
    bool store_o = true;
    if constexpr (TAIL) {
      int wf, wl;
      tile_parts(plan, tt, wf, wl);
      if (wf != wl) {
        constexpr int kSlotO = kThreads * T::NDB * 16;  // floats of O in one slot
        constexpr int kSlot = kSlotO + kThreads * 2;     // floats per slot
        // (the lane offsets are made opaque here, so that no address of this rarely run code is
        // computed ahead of the main loop and held in registers across it)
        uint32_t o_at = wave * T::NDB * 4 * 64 + lane;  // this lane's first 16-byte column
        uint32_t ml_at = kSlotO + (wave * 64 + lane) * 2;
        opaque(o_at);
        opaque(ml_at);
        int* const ctr = cnt + tt;
        const int others = wl - wf;
        if (tid == 0) s_last = __hip_atomic_load(ctr, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == others;
        __syncthreads();
        store_o = __builtin_amdgcn_readfirstlane(s_last) != 0;
        if (!store_o) {
          float* const mine = part + (size_t)tail_slot(w_tail, seg) * kSlot;
#pragma unroll
          for (int db = 0; db < T::NDB; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              *reinterpret_cast<f32x4*>(mine + (o_at + (db * 4 + jj) * 64) * 4) =
                  f32x4{oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
          *reinterpret_cast<u32x2*>(mine + ml_at) = u32x2{__float_as_uint(m_run), __float_as_uint(l_run)};
          __syncthreads();  // every wave's stores are done (in this XCD's L2)
          // arrive: publishes the stores device-wide (release: L2 write-back) and, for the last
          // part, makes the others' visible (acquire)
          if (tid == 0) s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == others;
          __syncthreads();
          store_o = __builtin_amdgcn_readfirstlane(s_last) != 0;
        }
        if (store_o) {
          // (thread 0's acquire above invalidated this CU's caches for every wave; the barrier
          // orders the loads below after it)
          auto slot_of = [&](int p) __attribute__((always_inline)) {
            return part + (size_t)tail_slot(p, tail_seg_of(plan, p, tt)) * kSlot;
          };
          // O = sum_p 2^(m_p - M) O_p and l = sum_p 2^(m_p - M) l_p over the parts in key
          // order, M the largest offset, formed as a running merge (the offset moves to the
          // larger of the two at each step; the same steps whichever part merges).  At D = 128
          // the channels are merged in two passes over the parts, so that the merged half, the
          // part being added and this part's own accumulator fit in registers together.
          constexpr int NP = T::NDB >= 4 ? 2 : 1;   // passes
          constexpr int DBP = T::NDB / NP;          // 32-channel blocks per pass
          float mm = -INFINITY, ml = 0.f;
#pragma unroll
          for (int pass = 0; pass < NP; ++pass) {
            f32x16 macc[DBP];
#pragma unroll
            for (int d = 0; d < DBP; ++d) macc[d] = f32x16{};
            float mrun = -INFINITY;
            for (int p = wf; p <= wl; ++p) {
              f32x16 x[DBP];
              float mp, lp;
              if (p == w_tail) {
#pragma unroll
                for (int d = 0; d < DBP; ++d) x[d] = oacc[pass * DBP + d];
                mp = m_run;
                lp = l_run;
              } else {
                const float* const slot = slot_of(p);
                const u32x2 ml2 = *reinterpret_cast<const u32x2*>(slot + ml_at);
                mp = __uint_as_float(ml2[0]);
                lp = __uint_as_float(ml2[1]);
#pragma unroll
                for (int d = 0; d < DBP; ++d)
#pragma unroll
                  for (int jj = 0; jj < 4; ++jj) {
                    const f32x4 v4 = *reinterpret_cast<const f32x4*>(
                        slot + (o_at + ((pass * DBP + d) * 4 + jj) * 64) * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[d][4 * jj + r] = v4[r];
                  }
              }
              const float M = fmaxf(mrun, mp);
              const float ea = __builtin_amdgcn_exp2f(mrun - M), eb = __builtin_amdgcn_exp2f(mp - M);
#pragma unroll
              for (int d = 0; d < DBP; ++d)
#pragma unroll
                for (int r = 0; r < 16; ++r) macc[d][r] = fmaf(x[d][r], eb, macc[d][r] * ea);
              if (pass == 0) ml = fmaf(lp, eb, ml * ea);
              mrun = M;
            }
#pragma unroll
            for (int d = 0; d < DBP; ++d) oacc[pass * DBP + d] = macc[d];
            mm = mrun;
          }
          l_run = ml;
          m_run = mm;
          // this tile's counter is not touched again in this launch: leave it zero for the next
          if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }

    // ---- epilogue: O = O_acc / l (fp32 or bf16), and optionally the row's log-sum-exp ------
    if (store_o) {
    const float l_tot = xor32_sum(l_run);
    const float inv = 1.f / l_tot;
    if constexpr (V8) {
      // the V codes' channel scales: lane holds channels 32 db + 8 jj + 4 hh + 0..3
#pragma unroll
      for (int db = 0; db < T::NDB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 sv = *reinterpret_cast<const f32x4*>(v_scale + (size_t)bh * D + 32 * db + 8 * jj + 4 * hh);
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[db][4 * jj + e] *= sv[e];
        }
    }
    if (q < Sq) {
      const int64_t orow = bb * a.osb + hd * a.osh + (int64_t)q * a.oss;  // element offset
      if (a.o_bf16) {
        uint16_t* o16 = reinterpret_cast<uint16_t*>(op) + orow;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const bf16x2 lo = {(__bf16)(oacc[db][4 * jj] * inv), (__bf16)(oacc[db][4 * jj + 1] * inv)};
            const bf16x2 hi = {(__bf16)(oacc[db][4 * jj + 2] * inv), (__bf16)(oacc[db][4 * jj + 3] * inv)};
            *reinterpret_cast<u32x2*>(o16 + db * 32 + 8 * jj + 4 * hh) =
                u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
          }
      } else {
        float* o32 = reinterpret_cast<float*>(op) + orow;
#pragma unroll
        for (int db = 0; db < T::NDB; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 o4 = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv,
                              oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv};
            *reinterpret_cast<f32x4*>(o32 + db * 32 + 8 * jj + 4 * hh) = o4;
          }
      }
      // log sum_j exp(scale * s_j) = (m + log2 l) * ln 2: the weights are 2^(scale log2e s - m)
      // (times 2^4 for fp8 V)
      if (lse != nullptr && hh == 0)
        lse[(int64_t)bh * Sq + q] =
            (m_run + __builtin_amdgcn_logf(l_tot) - (V8 ? kLog2WScale8 : 0.f)) * kLn2;
    }
    }
    if constexpr (TAIL) __syncthreads();  // the next segment refills the tile buffers
  }
}

// The tail workspace: kTailMaxG arrival counters, then two slots per tail workgroup, each the
// partial result of one part (every lane's O accumulator and its m, l) of 256 query rows.
constexpr size_t kTailCounterBytes = 1024;
static_assert(kTailCounterBytes >= kTailMaxG * sizeof(int), "tail counters");
constexpr size_t tail_slot_bytes(int D) { return (size_t)64 * 8 * (D / 2 + 2) * sizeof(float); }

// Zeroes the arrival counters of a split launch (a kernel rather than a memset, so the call can
// be captured into a graph).
__global__ void zero_counters_kernel(int* __restrict__ c, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) c[i] = 0;
}

// Position p of a 16-key step in a V^T row holds key vt_key(p): keys 0-3, 8-11, 4-7, 12-15,
// the order of the weights in the P^T operand (bits 2 and 3 swapped; an involution).
__device__ __forceinline__ int vt_key(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// V^T tiles of bf16 V at D = 128, for long sequences: tile t of (b, h) = bh holds the 64 keys
// the attention's key tile t covers (the last one the final 64 rows, as its K tile) as 128
// channel rows of 64 keys, vt[((bh * nkt + t) * 128 + channel) * 64 + position], each 16-key
// step in P^T order (vt_key), so that one 16-byte LDS read gives a lane the 8 keys of its half
// of a step; rows past S (only when S < 64) are zeros.  One workgroup per tile, through LDS.
__global__ __launch_bounds__(256) void vt_tiles_kernel(const uint16_t* __restrict__ v, Strides vs,
                                                        int H, int S, int nkt,
                                                        uint16_t* __restrict__ vt) {
  // 64 rows of 128 channels; the row pitch of 65 words puts the 8 rows a column read touches
  // in 8 distinct banks
  __shared__ uint32_t sm[64 * 65];
  const int bh = blockIdx.x / nkt, t = blockIdx.x - bh * nkt;
  const int r0 = t == nkt - 1 ? max(S - kBK, 0) : t * kBK;
  const uint16_t* vh = v + (bh / H) * vs.b + (bh % H) * vs.h;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;  // 16-byte chunk: row c / 16, channels 8 (c % 16) .. + 7
    const int row = c >> 4, ch8 = (c & 15) * 8;
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (r0 + row < S) x = *reinterpret_cast<const u32x4*>(vh + (int64_t)(r0 + row) * vs.s + ch8);
#pragma unroll
    for (int e = 0; e < 4; ++e) sm[row * 65 + ch8 / 2 + e] = x[e];
  }
  __syncthreads();
  uint16_t* out = vt + ((size_t)bh * nkt + t) * 128 * kBK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;  // output chunk: channel c / 8, positions 8 (c % 8) .. + 7
    const int ch = c >> 3, q = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int p0 = 8 * q + e;
      const int k0 = (p0 & ~15) | vt_key(p0 & 15), k1 = (p0 & ~15) | vt_key((p0 + 1) & 15);
      const uint32_t a0 = sm[k0 * 65 + ch / 2] >> (16 * (ch & 1));
      const uint32_t a1 = sm[k1 * 65 + ch / 2] >> (16 * (ch & 1));
      w[e / 2] = (a0 & 0xFFFFu) | (a1 << 16);
    }
    *reinterpret_cast<u32x4*>(out + ch * kBK + 8 * q) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Workgroups of the attention kernel resident at once on the stream's device: one per CU
// (8 wavefronts of two per SIMD), at most kTailMaxG.  Looked up once per device.
hipError_t resident_workgroups(hipStream_t stream, int& G) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g = cus < kTailMaxG ? cus : kTailMaxG;
    if (g < 1) return hipErrorInvalidDevice;
    cache[dev].store(g, std::memory_order_relaxed);
  }
  G = g;
  return hipSuccess;
}

template <int D, int KIND, int NW>
hipError_t launch(const AttnCall& ac, const void* q, Strides qs, const void* k, Strides ks,
                  const void* v, Strides vs, const float* q_scale, const float* k_scale,
                  const float* v_scale, hipStream_t stream) {
  using T = Tile<D, KIND != kBF16, NW, KIND == kFp8All>;
  KArgs a;
  a.qsb = qs.b; a.qsh = qs.h; a.qss = qs.s;
  a.ksb = ks.b; a.ksh = ks.h; a.kss = ks.s;
  a.vsb = vs.b; a.vsh = vs.h; a.vss = vs.s;
  a.osb = ac.os.b; a.osh = ac.os.h; a.oss = ac.os.s;
  a.H = ac.H;
  a.Sq = ac.Sq;
  a.Sk = ac.S;
  a.n_qt = (ac.Sq + T::BQ - 1) / T::BQ;
  a.c = ac.scale * kLog2e;
  a.o_bf16 = ac.o_bf16 ? 1 : 0;
  const int n_tiles = ac.B * ac.H * a.n_qt;  // (bounded by the shape checks of the C ABI)
  const int nkt = (ac.S + kBK - 1) / kBK;
  int G = 0;
  if (ac.tail != nullptr) {
    const hipError_t e = resident_workgroups(stream, G);
    if (e != hipSuccess) return e;
  }
  a.plan = split_plan(n_tiles, nkt, G);
  int* cnt = nullptr;
  float* part = nullptr;
  if (a.plan.n_tail > 0) {
    cnt = static_cast<int*>(ac.tail);
    part = reinterpret_cast<float*>(static_cast<uint8_t*>(ac.tail) + kTailCounterBytes);
    // the whole-tile launch zeroes the counters; without one, a kernel of its own does
    if (a.plan.n_main == 0)
      hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(256), 0, stream, cnt, a.plan.n_tail);
  }
  const uint8_t* qb = static_cast<const uint8_t*>(q);
  const uint8_t* kb = static_cast<const uint8_t*>(k);
  const uint8_t* vb = static_cast<const uint8_t*>(v);
  uint8_t* ob = static_cast<uint8_t*>(ac.o);
  auto attend = [&](auto vt_c) {
    constexpr bool VT = decltype(vt_c)::value;
    if (a.plan.n_main > 0)
      hipLaunchKernelGGL((attn_fwd_kernel<D, KIND, NW, false, VT>), dim3((unsigned)a.plan.n_main),
                         dim3(T::NT), 0, stream, qb, kb, vb, ob, ac.lse, q_scale, k_scale, v_scale,
                         part, cnt, a);
    if (a.plan.n_tail > 0)
      hipLaunchKernelGGL((attn_fwd_kernel<D, KIND, NW, true, VT>), dim3((unsigned)a.plan.G),
                         dim3(T::NT), 0, stream, qb, kb, vb, ob, ac.lse, q_scale, k_scale, v_scale,
                         part, cnt, a);
  };
  if constexpr (D == 128 && KIND != kFp8All) {
    if (ac.vt != nullptr) {
      // long sequences: V read through its V^T tiles (one 16-byte LDS read per product operand)
      hipLaunchKernelGGL(vt_tiles_kernel, dim3((unsigned)((long long)ac.B * ac.H * nkt)), dim3(256),
                         0, stream, static_cast<const uint16_t*>(v), vs, ac.H, ac.S, nkt,
                         static_cast<uint16_t*>(ac.vt));
      vb = static_cast<const uint8_t*>(ac.vt);
      attend(std::true_type{});
      return hipGetLastError();
    }
  }
  attend(std::false_type{});
  return hipGetLastError();
}

}  // namespace

size_t attn_vt_bytes(int B, int H, int S, int D) {
  if (D != 128 || S < kVtMinS) return 0;
  return (size_t)B * H * ((S + kBK - 1) / kBK) * (size_t)(128 * kBK * 2);
}

size_t attn_tail_bytes(int S, int D) {
  const int nkt = (S + kBK - 1) / kBK;
  // a tail needs ranges of kTailMinUnits key tiles, each shorter than a tile
  if (nkt <= kTailMinUnits || (D != 64 && D != 128)) return 0;
  return kTailCounterBytes + 2 * (size_t)kTailMaxG * tail_slot_bytes(D);
}

// Waves per workgroup.  Eight waves (256 query rows; one workgroup per CU, two waves per
// SIMD) share each K/V tile twice as widely as four, halving the L2 -> LDS traffic per flop;
// measured 4-6% faster on both variants at S = 4608 and S = 118800.
constexpr int kWaves = 8;

hipError_t launch_attn_bf16(const AttnCall& ac, hipStream_t stream) {
  if (ac.D == 64)
    return launch<64, kBF16, kWaves>(ac, ac.q, ac.qs, ac.k, ac.ks, ac.v, ac.vs, nullptr, nullptr,
                                     nullptr, stream);
  return launch<128, kBF16, kWaves>(ac, ac.q, ac.qs, ac.k, ac.ks, ac.v, ac.vs, nullptr, nullptr,
                                    nullptr, stream);
}

hipError_t launch_attn_int8(const AttnCall& ac, const int8_t* q_codes, const int8_t* k_codes,
                            const float* q_scale, const float* k_scale, hipStream_t stream) {
  // the codes are the prepass's own contiguous [B, H, S, D] buffers
  const Strides cs{(int64_t)ac.H * ac.S * ac.D, (int64_t)ac.S * ac.D, ac.D};
  if (ac.D == 64)
    return launch<64, kInt8, kWaves>(ac, q_codes, cs, k_codes, cs, ac.v, ac.vs, q_scale, k_scale,
                                     nullptr, stream);
  return launch<128, kInt8, kWaves>(ac, q_codes, cs, k_codes, cs, ac.v, ac.vs, q_scale, k_scale,
                                    nullptr, stream);
}

hipError_t launch_attn_fp8(const AttnCall& ac, const uint8_t* q_codes, const uint8_t* k_codes,
                           const float* q_scale, const float* k_scale, hipStream_t stream) {
  const Strides cs{(int64_t)ac.H * ac.S * ac.D, (int64_t)ac.S * ac.D, ac.D};
  if (ac.D == 64)
    return launch<64, kFp8, kWaves>(ac, q_codes, cs, k_codes, cs, ac.v, ac.vs, q_scale, k_scale,
                                    nullptr, stream);
  return launch<128, kFp8, kWaves>(ac, q_codes, cs, k_codes, cs, ac.v, ac.vs, q_scale, k_scale,
                                   nullptr, stream);
}

hipError_t launch_attn_fp8_all(const AttnCall& ac, const uint8_t* q_codes, const uint8_t* k_codes,
                               const uint8_t* v_codes, const float* q_scale, const float* k_scale,
                               const float* v_scale, hipStream_t stream) {
  if (ac.D != 128) return hipErrorInvalidValue;
  const Strides cs{(int64_t)ac.H * ac.S * ac.D, (int64_t)ac.S * ac.D, ac.D};
  return launch<128, kFp8All, kWaves>(ac, q_codes, cs, k_codes, cs, v_codes, cs, q_scale, k_scale,
                                      v_scale, stream);
}

}  // namespace ditattn
