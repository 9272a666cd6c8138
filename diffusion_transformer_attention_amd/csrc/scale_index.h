// Which per-block quantization scale the 8-bit attention kernels read.  Plain integer
// arithmetic, compiled for the device by the kernels and for the host by a test that replays it
// over every query tile and key tile of ragged sequence lengths.
#pragma once

#include <hip/hip_runtime.h>

namespace ditattn {

constexpr int kScaleQBlock = 128;  // tokens per Q scale block
constexpr int kScaleKBlock = 64;   // tokens per K scale block (= one key tile)
constexpr int kRowsPerWave = 32;   // query rows owned by one wavefront

// Q scale block of the rows of wavefront `wave` in query tile `qt` (tiles of `bq` rows), for a
// sequence with `nqb` Q blocks.  A wavefront whose rows all lie past the end of the sequence
// (in a ragged last tile) computes nothing it stores, but its scale is still loaded: the index
// is clamped to the last block so that the load stays inside this (b, h)'s scale segment.
__host__ __device__ inline int q_scale_block(int qt, int wave, int bq, int nqb) {
  const int blk = (qt * bq + wave * kRowsPerWave) / kScaleQBlock;
  return blk < nqb ? blk : nqb - 1;
}

// K scale block of key tile `jt` out of `nkt` tiles.  The software pipeline evaluates one tile
// past the last (its results are discarded), so `jt` may reach nkt; it is clamped likewise.
__host__ __device__ inline int k_scale_block(int jt, int nkt) { return jt < nkt - 1 ? jt : nkt - 1; }

}  // namespace ditattn
