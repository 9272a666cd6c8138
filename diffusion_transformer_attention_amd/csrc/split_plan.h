// How an attention launch shares out its last, partly filled round of query tiles.
//
// A launch has n_tiles query tiles (256 rows of one (b, h) each) of nkt key tiles (64 keys)
// each; one (query tile, key tile) pair is one unit of work.  With G workgroups resident at once
// (one per CU), the first n_main = G floor(n_tiles / G) tiles fill whole rounds and run one
// workgroup per tile.  The n_tail tiles left over would leave CUs idle in a last round; instead
// their units, in (tile, key tile) order, are cut into G contiguous ranges of equal length (to
// one unit), one workgroup each — the data-parallel plus stream-K hybrid of split GEMMs, here
// over the key axis of attention.  A range is shorter than a tile, so it holds the end of one
// tile and the start of the next at most: a workgroup has one or two segments, and the segments
// on one tile, from consecutive workgroups, are its parts.  Each part leaves its partial result
// (unnormalised O, offset m and sum l of every row) in a workspace slot, and whichever part of a
// tile finishes last merges them in part order, so the result does not depend on timing.
//
// Plain integer arithmetic, compiled for the device by the kernel, for the host by the launcher
// and by a test that checks it exhaustively on small shapes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

constexpr int kTailMaxG = 256;     // most workgroups a tail is shared among (CUs of an MI355X)
constexpr int kTailMinUnits = 8;   // no tail phase when a range would be shorter than this
// No tail phase either when the last round would keep more than 5/8 of the CUs busy.  The
// chip is power limited: a round that leaves a few CUs idle runs at a higher clock and is
// nearly as fast as a full one, and the shared-out tiles cost more per unit of work (partial
// results, and the tail launch's own, slower schedule).  Measured on bf16 launches: +11% at
// 9/16 busy (B1 H8 S4608), +1.3% at 5/8, break-even at 11/16, -5.6% at 27/32.
constexpr int kTailMaxFill8 = 5;   // eighths of G

struct SplitPlan {
  int n_main;   // query tiles run whole, by workgroups 0 .. n_main - 1
  int n_tail;   // query tiles shared out among workgroups n_main .. n_main + G - 1 (0: none)
  int G;        // tail workgroups (0 when n_tail = 0)
  int nkt;      // key tiles per query tile
  int64_t U;    // tail units: n_tail * nkt
};

// The plan for n_tiles query tiles of nkt key tiles on G resident workgroups (G <= kTailMaxG).
// No tail phase when the tiles fill whole rounds, a range would be shorter than kTailMinUnits
// or the last round is more than kTailMaxFill8 / 8 full.
__host__ __device__ inline SplitPlan split_plan(int n_tiles, int nkt, int G) {
  SplitPlan p;
  p.nkt = nkt;
  p.n_main = G > 0 ? (n_tiles / G) * G : n_tiles;
  p.n_tail = n_tiles - p.n_main;
  p.G = G;
  p.U = (int64_t)p.n_tail * nkt;
  if (p.n_tail == 0 || p.U < (int64_t)kTailMinUnits * G || 8 * p.n_tail > kTailMaxFill8 * G) {
    p.n_main = n_tiles;
    p.n_tail = 0;
    p.G = 0;
    p.U = 0;
  }
  return p;
}

// First unit of tail workgroup w; w = G gives U.
__host__ __device__ inline int64_t tail_lo(const SplitPlan& p, int w) {
  return (int64_t)w * p.U / p.G;
}

// The tail workgroup whose range holds unit u (0 <= u < U): the largest w with tail_lo(w) <= u.
__host__ __device__ inline int tail_wg_of_unit(const SplitPlan& p, int64_t u) {
  const int64_t w = ((u + 1) * p.G - 1) / p.U;
  return (int)(w < p.G - 1 ? w : p.G - 1);
}

// Segment s (0 or 1) of tail workgroup w: tail tile t (0-based among the tail tiles) and its
// key tiles [k0, k1).  False when the workgroup has no such segment.  Segment 0 always exists
// and ends a tile (k1 = nkt) unless the range lies inside one tile; segment 1, when there is
// one, starts the next tile (k0 = 0).
//
// A workgroup runs segment 1 before segment 0.  Every range has the same length n (to one
// unit), so at time tau (in key tiles) each tail workgroup is at key tile tau of its segment
// 1, or, once that is done, at key tile tau + nkt - n of its segment 0, which ends with the
// range: all of them are at the same key tile (to within one) and those of one (b, h) share
// each K and V tile in their XCD's L2 as whole tiles do.  The part that ends its tile last,
// and merges it, is then the segment 0 part, at the end of the launch.
__host__ __device__ inline bool tail_segment(const SplitPlan& p, int w, int s, int& t, int& k0,
                                             int& k1) {
  const int64_t lo = tail_lo(p, w), hi = tail_lo(p, w + 1);
  const int64_t tt = lo / p.nkt + s;
  if (hi <= lo || tt * p.nkt >= hi) return false;
  const int64_t a = lo > tt * p.nkt ? lo : tt * p.nkt;
  const int64_t b = hi < (tt + 1) * p.nkt ? hi : (tt + 1) * p.nkt;
  t = (int)tt;
  k0 = (int)(a - tt * p.nkt);
  k1 = (int)(b - tt * p.nkt);
  return true;
}

// The tail workgroups holding the parts of tail tile t, in key order: w_first .. w_last.
__host__ __device__ inline void tile_parts(const SplitPlan& p, int t, int& w_first, int& w_last) {
  w_first = tail_wg_of_unit(p, (int64_t)t * p.nkt);
  w_last = tail_wg_of_unit(p, (int64_t)(t + 1) * p.nkt - 1);
}

// Which segment of tail workgroup w lies on tail tile t (w one of the tile's workgroups).
__host__ __device__ inline int tail_seg_of(const SplitPlan& p, int w, int t) {
  return (int)(t - tail_lo(p, w) / p.nkt);
}

// The work item that dispatch slot i of n takes.  The dispatcher sends workgroup i to XCD
// i % 8; this order gives each XCD a contiguous range of items, so the workgroups sharing one
// XCD's L2 work on consecutive query tiles (or tail ranges) of the same (b, h) and stream the
// same K and V tiles.  Whole tile of workgroup wg < n_main: xcd_order(wg, n_main); tail
// workgroup of workgroup n_main + j: xcd_order(j, G) (n_main is a multiple of G).
__host__ __device__ inline int xcd_order(int i, int n) {
  const int per = n >> 3, rem = n & 7, xcd = i & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + (i >> 3);
}

// Workspace slot of segment s of tail workgroup w: two per workgroup.
__host__ __device__ inline int tail_slot(int w, int s) { return 2 * w + s; }

}  // namespace ditattn
