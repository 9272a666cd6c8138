"""Mutation check of the oracle's pins (run by hand: python tests/oracle_mutations.py).

Each entry plants one plausible mistake in a copy of oracle/ (a dropped term, a wrong sign,
index or constant, a changed rounding rule) and runs the CPU pins on the copy; every mistake
must make them fail.  It copies oracle/, datagen/ and tests/ to a temporary folder and never
touches the repository.  Not collected by pytest (the file name does not start with test_).
"""
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle.py", "tests/test_oracle_fp8.py", "tests/test_oracle_fbcache.py"]

# (file, text, replacement): the definitions of the core path
CORE = [
 ("oracle/attention.py", "w = np.exp(s - s.max(axis=1, keepdims=True))", "w = np.exp(s)"),
 ("oracle/attention.py", "s = (q[r0:r0 + _ROW_CHUNK] @ kt) * scale", "s = (q[r0:r0 + _ROW_CHUNK] @ kt) * scale * 1.0001"),
 ("oracle/attention.py", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D"),
 ("oracle/attention.py", "/ w.sum(axis=1, keepdims=True)", "/ w.sum(axis=1, keepdims=True).mean()"),
 ("oracle/quant.py", "q = np.rint(blk / scale[:, :, None, None])", "q = np.round(blk / scale[:, :, None, None] + 1e-7)"),
 ("oracle/quant.py", "scale = amax / np.float32(QMAX)", "scale = amax * (np.float32(1) / np.float32(QMAX))"),
 ("oracle/quant.py", "sq_rows = np.asarray(q_scale, dtype=np.float64)[:, :, rows // q_block]", "sq_rows = np.asarray(q_scale, dtype=np.float64)[:, :, np.minimum(rows // k_block, q_scale.shape[2]-1)]"),
 ("oracle/quant.py", "out[b, h, d] = np.float32(math.fsum(cols[d].tolist()) / S)", "out[b, h, d] = np.float32(cols[d].sum() / S)"),
 ("oracle/quant.py", "return kf - np.asarray(kmean, dtype=np.float32)[:, :, None, :]", "return kf + np.asarray(kmean, dtype=np.float32)[:, :, None, :]"),
 ("oracle/quant.py", "return np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)", "return scale.astype(np.float32)"),
 ("oracle/rel_l1.py", "den = np.abs(b).sum()", "den = np.abs(a).sum()"),
 ("oracle/rel_l1.py", "num = np.abs(a - b).sum()", "num = np.abs(a + b).sum()"),
]


# the NEXT rows: log-sum-exp, fp8, probe, First Block Cache
NEXT = [
 # log-sum-exp
 ("oracle/attention.py", "out[b, h, r0:r0 + _ROW_CHUNK] = m + np.log(", "out[b, h, r0:r0 + _ROW_CHUNK] = np.log(np.exp(m)) * 0 + m * 1.0 + 0.001 + np.log("),
 ("oracle/quant.py", "out[b, h, r0:r0 + 1024] = m + np.log(np.exp(sc - m[:, None]).sum(axis=1))", "out[b, h, r0:r0 + 1024] = m + np.log(np.exp(sc - m[:, None]).mean(axis=1))"),
 # fp8 format
 ("oracle/quant.py", "(1.0 + m / 8.0) * 2.0 ** (e - 7.0)", "(1.0 + m / 8.0) * 2.0 ** (e - 8.0)"),
 ("oracle/quant.py", "m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
 ("oracle/quant.py", "mag = np.where((e == 15) & (m == 7), np.nan, mag)", "mag = np.where((e == 15) & (m >= 6), np.nan, mag)"),
 ("oracle/quant.py", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
 ("oracle/quant.py", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo))"),
 ("oracle/quant.py", "np.where(np.signbit(x), 0x80, 0)", "np.where(x < 0, 0x80, 0)"),
 ("oracle/quant.py", "E4M3_MAX = 448.0", "E4M3_MAX = 480.0"),
 # fp8 quantizers
 ("oracle/quant.py", "        scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)\n        scales[:, :, t] = scale",
                     "        scale = np.where(amax == 0, np.float32(1.0), (amax * np.float32(1 / E4M3_MAX))).astype(np.float32)\n        scales[:, :, t] = scale"),
 ("oracle/quant.py", "    kc, ks = quantize_blocks_fp8(smooth_k(k, kmean), K_BLOCK)", "    kc, ks = quantize_blocks_fp8(np.asarray(k, dtype=np.float32), K_BLOCK)"),
 ("oracle/quant.py", "    amax = np.abs(x).max(axis=2)                                            # [B, H, D]", "    amax = np.abs(x).max(axis=(2, 3), keepdims=False)[:, :, None] + 0 * np.abs(x).max(axis=2)"),
 ("oracle/quant.py", "    vq = e4m3_value(v_codes) * np.asarray(v_scale, dtype=np.float64)[:, :, None, :]", "    vq = e4m3_value(v_codes) * np.asarray(v_scale, dtype=np.float64)[:, :, None, :].mean()"),
 # probe
 ("oracle/quant.py", "    return step // 2 + np.arange(n_rows, dtype=np.int64) * step", "    return (step - 1) // 2 + np.arange(n_rows, dtype=np.int64) * step"),
 ("oracle/quant.py", "    return float(np.sqrt(num.sum() / den.sum())), np.sqrt(num / den)", "    return float(np.sqrt(num / den).mean()), np.sqrt(num / den)"),
 # First Block Cache
 ("oracle/fbcache.py", "    if diff is None or not (d < thr):", "    if diff is None or not (d <= thr):"),
 ("oracle/fbcache.py", "    if state.steps < cfg.max_warmup_steps:", "    if state.steps <= cfg.max_warmup_steps:"),
 ("oracle/fbcache.py", "state.cached_steps >= cfg.max_cached_steps:", "state.cached_steps > cfg.max_cached_steps:"),
 ("oracle/fbcache.py", "state.continuous >= cfg.max_continuous_cached_steps:", "state.continuous > cfg.max_continuous_cached_steps:"),
 ("oracle/fbcache.py", "                        continuous=state.continuous + 1 if use else 0,", "                        continuous=state.continuous + 1,"),
 ("oracle/fbcache.py", "        if not state.use_cache:\n            prev = r", "        prev = r"),
 ("oracle/fbcache.py", "    keep_odd = (bits >> np.uint64(45)) & np.uint64(1)", "    keep_odd = np.uint64(0) * bits"),
 ("oracle/fbcache.py", "    return bf16_round(_bf16_value(a_bits) - _bf16_value(b_bits))", "    return bf16_round(_bf16_value(b_bits) - _bf16_value(a_bits))"),
 ("oracle/fbcache.py", "    sub = np.rint(x * 2.0 ** 133) * 2.0 ** -133", "    sub = np.trunc(x * 2.0 ** 133) * 2.0 ** -133"),
]



def main() -> int:
    missed = []
    for f, old, new in CORE + NEXT:
        tmp = tempfile.mkdtemp()
        try:
            for d in ("oracle", "datagen", "tests"):
                shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d))
            path = os.path.join(tmp, f)
            src = open(path).read()
            assert old in src, (f, old)
            open(path, "w").write(src.replace(old, new))
            r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", *PINS, "-m", "not gpu",
                                "-p", "no:cacheprovider"], cwd=tmp, capture_output=True, text=True)
        finally:
            shutil.rmtree(tmp)
        caught = r.returncode != 0
        print("caught" if caught else "MISSED", f, new.strip()[:70], flush=True)
        if not caught:
            missed.append((f, new))
    print(f"{len(CORE) + len(NEXT) - len(missed)} of {len(CORE) + len(NEXT)} caught")
    return 1 if missed else 0


if __name__ == "__main__":
    sys.exit(main())
