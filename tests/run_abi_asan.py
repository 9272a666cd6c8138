"""Run the C ABI checks (tests/test_abi.py) on a host-instrumented build (AddressSanitizer).

CPU only; no GPU is touched.  The library's host layer (csrc/capi.hip: argument validation,
workspace sizes and offsets, the launch set-up) is compiled with AddressSanitizer for the host
pass only, linked with the ordinary objects of the kernel sources into
_build/asan/libditattn_asan.so, and tests/test_abi.py then drives every entry point's
validation and workspace arithmetic through it, with the sanitizer runtime preloaded into the
Python process.  Any out-of-bounds access, use after free or similar in the host code aborts
the run with a sanitizer report.

    python tests/run_abi_asan.py          (exit status 0: clean)
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from diffusion_transformer_attention_amd import build as libbuild  # noqa: E402


def main() -> int:
    libbuild.build()  # the ordinary objects of every source, in _build/
    hipcc = libbuild._hipcc()
    out_dir = os.path.join(libbuild.BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "capi.o")
    lib = os.path.join(out_dir, "libditattn_asan.so")
    # host pass instrumented; the device code of capi.hip (none) and of the kernels is not
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.run([hipcc, *libbuild.FLAGS, "-O1", "-g", *san, "-I", libbuild.CSRC, "-c",
                    os.path.join(libbuild.CSRC, "capi.hip"), "-o", obj], check=True)
    others = [os.path.join(libbuild.BUILD, n) for n in sorted(os.listdir(libbuild.BUILD))
              if n.endswith(".o") and n != "capi.o"]
    subprocess.run([hipcc, f"--offload-arch={libbuild.ARCH}", "-shared", "-fPIC",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan",
                    "-o", lib, obj, *others], check=True)
    rt = subprocess.run([os.path.join(os.path.dirname(hipcc), "..", "llvm", "bin", "clang"),
                         "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=rt, DITATTN_ABI_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    print(f"sanitizer runtime {rt}\nlibrary {lib}", flush=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], env=env)
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
