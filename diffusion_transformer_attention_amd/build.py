"""Build libditattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage:  python -m diffusion_transformer_attention_amd.build   (or call build()).

Every HIP source under csrc/ is compiled with hipcc for gfx950 (one process per file, in
parallel), then linked into diffusion_transformer_attention_amd/libditattn.so.  Object files
go to _build/ at the repository root.  Packed fp32 VALU instructions are disabled in device
code (``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does not know
that feature, which is harmless.
"""
from __future__ import annotations

import glob
import json
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libditattn.so")
BUILD_INFO = os.path.join(PKG, "build_info.json")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libditattn.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libditattn.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = [[hipcc, *FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


def _write_build_info() -> None:
    """Record which source revision the library was built from (the benchmark reports it; the
    GPU machine that runs the benchmark has the built tree but not its git history)."""
    def git(*args):
        try:
            r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=30)
            return r.stdout.strip() if r.returncode == 0 else None
        except (OSError, subprocess.SubprocessError):
            return None
    sha = git("rev-parse", "HEAD")
    status = git("status", "--porcelain", "--untracked-files=no")
    info = {"git_sha": sha, "dirty": bool(status) if status is not None else None}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    print(build(verbose=True))
