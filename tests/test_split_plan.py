"""How the attention kernel shares out its last round of query tiles, replayed on the host (CPU).

The kernel takes every decision about which workgroup computes which keys of which query tile
from ``csrc/split_plan.h``.  This test compiles that same header into a host program and
checks, over every plan of small shapes (all tile counts up to several rounds, key-tile counts
1..40, 1..9 and 16/32/256 resident workgroups) and the plans of the workload shapes:

* the whole tiles and the tail tiles together are every tile once;
* the tail workgroups' segments, in workgroup and segment order, are every tail unit (query
  tile, key tile) exactly once and in order, each workgroup holding at most two non-empty
  segments of at least the minimum length in total;
* the parts the merge looks up for a tile (its first and last workgroup and the segment index
  within each) are exactly the segments found on that tile, and their slots are distinct;
* a workgroup with two segments has its second start a tile (key tile 0) and its first end the
  previous one (key tile nkt), and every range has the same length to one unit: run second
  segment first, all tail workgroups are at the same key tile (to within one) at any time;
* the XCD remaps of the whole tiles and of the tail workgroups are permutations.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "diffusion_transformer_attention_amd", "csrc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")

PROGRAM = r"""
#include <cstdio>
#include <vector>
#include "split_plan.h"
using namespace ditattn;

static long checked = 0;

#define FAIL(...) do { printf(__VA_ARGS__); printf("  [n_tiles=%d nkt=%d G=%d]\n", n_tiles, nkt, G); return false; } while (0)

static bool check(int n_tiles, int nkt, int G) {
  const SplitPlan p = split_plan(n_tiles, nkt, G);
  if (p.n_main + p.n_tail != n_tiles) FAIL("tiles lost");
  // the whole tiles and the tail workgroups: the remaps are permutations
  if (G > 0) {
    std::vector<char> seen(G, 0);
    for (int j = 0; j < G; ++j) {
      const int w = xcd_order(j, G);
      if (w < 0 || w >= G || seen[w]) FAIL("tail remap not a permutation at %d", j);
      seen[w] = 1;
    }
  }
  {
    std::vector<char> seen(p.n_main, 0);
    for (int wg = 0; wg < p.n_main; ++wg) {
      const int t = xcd_order(wg, p.n_main);
      if (t < 0 || t >= p.n_main || seen[t]) FAIL("remap not a permutation at wg %d", wg);
      seen[t] = 1;
    }
  }
  if (p.n_tail == 0) {
    if (p.G != 0 || p.U != 0) FAIL("empty tail with G or U set");
    // no tail although one was possible: only when the ranges would be too short
    const int full = G > 0 ? (n_tiles / G) * G : n_tiles;
    if (full != n_tiles && (long long)(n_tiles - full) * nkt >= (long long)kTailMinUnits * G &&
        8 * (n_tiles - full) <= kTailMaxFill8 * G)
      FAIL("tail phase skipped");
    return true;
  }
  if (p.n_main % p.G != 0 || p.n_tail >= p.G || p.G != G) FAIL("bad split of tiles");
  if (8 * p.n_tail > kTailMaxFill8 * G) FAIL("tail phase for a last round %d of %d full", p.n_tail, G);
  if (p.U != (int64_t)p.n_tail * nkt) FAIL("bad U");
  // walk the segments in order
  int64_t cursor = 0;
  std::vector<int> first_w(p.n_tail, -1), last_w(p.n_tail, -1);
  std::vector<std::vector<int>> seg_w(p.n_tail), seg_s(p.n_tail);
  std::vector<char> slot_used(2 * G, 0);
  const int64_t n_lo = p.U / G, n_hi = (p.U + G - 1) / G;
  for (int w = 0; w < G; ++w) {
    int64_t len = 0;
    {
      int t0, a0, b0, t1, a1, b1;
      tail_segment(p, w, 0, t0, a0, b0);
      if (tail_segment(p, w, 1, t1, a1, b1) && (a1 != 0 || b0 != nkt || t1 != t0 + 1))
        FAIL("wg %d: segments [%d,%d) of %d and [%d,%d) of %d", w, a0, b0, t0, a1, b1, t1);
    }
    for (int s = 0; s < 3; ++s) {
      int t = -1, k0 = -1, k1 = -1;
      const bool has = tail_segment(p, w, s, t, k0, k1);
      if (s == 2) {
        if (has) FAIL("third segment in wg %d", w);
        break;
      }
      if (!has) {
        if (s == 0) FAIL("wg %d has no segment", w);
        continue;
      }
      if (t < 0 || t >= p.n_tail || k0 < 0 || k1 <= k0 || k1 > nkt) FAIL("bad segment %d/%d: t=%d [%d,%d)", w, s, t, k0, k1);
      if ((int64_t)t * nkt + k0 != cursor) FAIL("segment %d/%d does not continue the previous one", w, s);
      cursor = (int64_t)t * nkt + k1;
      len += k1 - k0;
      if (first_w[t] < 0) first_w[t] = w;
      last_w[t] = w;
      seg_w[t].push_back(w);
      seg_s[t].push_back(s);
      const int slot = tail_slot(w, s);
      if (slot < 0 || slot >= 2 * kTailMaxG || slot_used[slot]) FAIL("slot %d reused", slot);
      slot_used[slot] = 1;
      ++checked;
    }
    if (len < kTailMinUnits) FAIL("wg %d range of %lld units", w, (long long)len);
    if (len < n_lo || len > n_hi) FAIL("wg %d range of %lld units, not %lld..%lld", w, (long long)len, (long long)n_lo, (long long)n_hi);
    if (cursor != tail_lo(p, w + 1)) FAIL("wg %d range does not end at the next start", w);
  }
  if (cursor != p.U) FAIL("units not all covered");
  for (int t = 0; t < p.n_tail; ++t) {
    int wf = -1, wl = -1;
    tile_parts(p, t, wf, wl);
    if (wf != first_w[t] || wl != last_w[t]) FAIL("tile %d parts %d..%d, segments in %d..%d", t, wf, wl, first_w[t], last_w[t]);
    if ((int)seg_w[t].size() != wl - wf + 1) FAIL("tile %d: a workgroup in %d..%d holds no part", t, wf, wl);
    for (size_t i = 0; i < seg_w[t].size(); ++i) {
      if (seg_w[t][i] != wf + (int)i) FAIL("tile %d parts not consecutive", t);
      if (tail_seg_of(p, seg_w[t][i], t) != seg_s[t][i]) FAIL("tile %d: segment index of wg %d", t, seg_w[t][i]);
    }
  }
  return true;
}

int main() {
  const int gs[] = {1, 2, 3, 4, 5, 6, 7, 8, 9, 16, 32, 256};
  for (int G : gs)
    for (int nkt = 1; nkt <= 40; ++nkt)
      for (int n_tiles = 1; n_tiles <= 3 * G + 5; ++n_tiles)
        if (!check(n_tiles, nkt, G)) return 1;
  // the workload shapes: B1 / B2 H24 S4608, B2 H24 S11440, B1 H24 S118800, D = 128 (256-row
  // tiles), and a few with little work in the tail
  struct W { int n_tiles, nkt; } ws[] = {{432, 72}, {864, 72}, {2160, 179}, {11160, 1857},
                                         {24 * 513, 2049}, {255, 100000}, {257, 100000}};
  for (const W& w : ws)
    for (int G : {256, 255, 128, 80, 32})
      if (!check(w.n_tiles, w.nkt, G)) return 1;
  printf("ok %ld\n", checked);
  return 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_split_plan_covers_every_unit_once(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "plan.cpp"
    exe = tmp_path / "plan"
    src.write_text(PROGRAM)
    # host-only compilation of the kernel's own header (no device code is generated)
    r = subprocess.run([hipcc, "-x", "c++", "-O1", "-std=c++17", "-I", CSRC, "-I", ROCM_INCLUDE,
                        "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
