"""The 8-bit attention kernels' scale indexing, replayed on the host (CPU only).

The kernels take the index of the Q and K quantization scale they load from
``csrc/scale_index.h``.  This test compiles that same header into a host program and walks it
over every query tile, wavefront and key tile the kernel's grid covers, for ragged sequence
lengths and the workload lengths: every index must lie inside the (b, h) segment of its scale
array, and a wavefront that owns rows of the sequence must read the scale of their block.
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
#include "scale_index.h"
using namespace ditattn;

int main() {
  long checked = 0;
  int lengths[2100];
  int n = 0;
  for (int s = 1; s <= 2048; ++s) lengths[n++] = s;
  const int extra[] = {4608, 11440, 118800, 118801, 131071, 131072};
  for (int s : extra) lengths[n++] = s;
  for (int waves : {4, 8}) {
    const int bq = kRowsPerWave * waves;
    for (int i = 0; i < n; ++i) {
      const int S = lengths[i];
      const int nqb = (S + kScaleQBlock - 1) / kScaleQBlock;
      const int nkt = (S + kScaleKBlock - 1) / kScaleKBlock;
      const int n_qt = (S + bq - 1) / bq;
      for (int qt = 0; qt < n_qt; ++qt)
        for (int w = 0; w < waves; ++w) {
          const int idx = q_scale_block(qt, w, bq, nqb);
          if (idx < 0 || idx >= nqb) {
            printf("q index %d outside [0, %d): S=%d waves=%d qt=%d wave=%d\n", idx, nqb, S, waves, qt, w);
            return 1;
          }
          const int r0 = qt * bq + w * kRowsPerWave;  // first row of the wavefront
          if (r0 < S) {
            const int r1 = (r0 + kRowsPerWave < S ? r0 + kRowsPerWave : S) - 1;
            if (idx != r0 / kScaleQBlock || idx != r1 / kScaleQBlock) {
              printf("rows %d..%d read block %d: S=%d\n", r0, r1, idx, S);
              return 1;
            }
          }
          ++checked;
        }
      for (int jt = 0; jt <= nkt; ++jt) {  // one tile past the end, as the pipeline does
        const int idx = k_scale_block(jt, nkt);
        if (idx < 0 || idx >= nkt || (jt < nkt && idx != jt)) {
          printf("k index %d for tile %d of %d: S=%d\n", idx, jt, nkt, S);
          return 1;
        }
        ++checked;
      }
    }
  }
  printf("ok %ld\n", checked);
  return 0;
}
"""


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_scale_indices_stay_in_segment(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "replay.cpp"
    exe = tmp_path / "replay"
    src.write_text(PROGRAM)
    # host-only compilation of the kernels' own header (no device code is generated)
    r = subprocess.run([hipcc, "-x", "c++", "-O1", "-std=c++17", "-I", CSRC, "-I", ROCM_INCLUDE,
                        "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok ")
