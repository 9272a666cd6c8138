"""Benchmark of the DiT attention hot path on one MI355X.

One step = the whole path once over one batch of resident synthetic input:
  attn_fwd_bf16    B=1 H=24 S=118800 D=128 (a 720p 129-frame video latent)
  attn_fwd_int8qk  same tensors (K mean, int8 quantization and int8-QK attention)
  resid_rel_l1     two bf16 [118800, 3072] first-block residuals
Throughput counts 4*B*H*S^2*D flops per attention call; `value` is the counted flops of both
attention calls per step divided by the step time (the rel-L1 pass is inside the step).
The image-DiT shape (S=4608) is timed after the main loop and reported in `extra`.

Prints ONE JSON line.  Options: --gpus N (only 1: this build runs on one GPU),
--steps K, --warmup W, --no-cpu-baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
# The int8-QK call does half its counted flops (QK) on int8 MFMA and half (PV) on bf16 MFMA, so
# even at both peaks it reaches only 1 / (0.5 / 5000 + 0.5 / 2500) = 3333 TOPS (66.7% of int8).
PEAK_INT8_BF16PV_TOPS = 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_BF16_TFLOPS)
ATTN_KERNEL = "attn_fwd_kernel<128, 0, 8>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_longvideo_traffic.json")


def attn_flops(B, H, S, D):
    return 4.0 * B * H * S * S * D


def make_inputs(torch, B, H, S, D, seed, koff_var=2.0):
    """Seeded synthetic Q, K, V on the GPU: N(0,1), K plus a per-(h, d) offset ~ N(0, var)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shape = (B, H, S, D)
    q = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    off = math.sqrt(koff_var) * torch.randn((1, H, 1, D), generator=g, device="cuda")
    k = (torch.randn(shape, generator=g, device="cuda") + off).to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    return q, k, v


def make_residuals(torch, rows, cols, seed, noise=0.05):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    b = torch.randn((rows, cols), generator=g, device="cuda").to(torch.bfloat16)
    a = (b.float() + noise * torch.randn((rows, cols), generator=g, device="cuda")).to(torch.bfloat16)
    return a, b


def kernel_source_hash():
    h = hashlib.sha256()
    for name in ("attn_fwd.hip", "device_common.h"):
        with open(os.path.join(ROOT, "diffusion_transformer_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch of the bf16 attention kernel, from committed rocprofv3 counters,
    or None if they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(budget_s=15.0):
    """The fp64 oracle timed on the host cores on a bounded sample of the step's workload:
    exact attention for a few query rows of one head at S=118800 (all keys), plus the
    relative-L1 reduction over a slice of the residuals."""
    import numpy as np
    import datagen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = len(os.sched_getaffinity(0))
    S, D = 118800, 128
    wid = datagen.WORKLOADS["longvideo"][0]
    off = datagen.k_offsets(wid, 1, D, 2.0)
    q, k, v = datagen.qkv_head(wid, 0, 0, S, D, off[0])
    qf, kf, vf = (datagen.bf16_to_f64(t)[None, None] for t in (q, k, v))
    rows, total_rows, t_attn = 32, 0, 0.0
    while t_attn < budget_s * 0.8:
        sel = np.arange(total_rows, total_rows + rows) % S
        t0 = time.perf_counter()
        oracle.attention_rows(qf, kf, vf, sel)
        t_attn += time.perf_counter() - t0
        total_rows += rows
        rows = min(rows * 2, 4096)
    tflops = 4.0 * total_rows * S * D / t_attn / 1e12
    # the int8-QK oracle on the same head: K mean, codes and scales for the whole head, then
    # attention on the codes for a block of query rows
    t0 = time.perf_counter()
    qq = oracle.quantize_qk(qf, kf)
    t_quant = time.perf_counter() - t0
    rows8 = 1024
    t0 = time.perf_counter()
    oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], vf,
                          rows=np.arange(rows8))
    t_int8 = time.perf_counter() - t0
    a, b = datagen.residual_pair(4096, 3072)
    af, bf = datagen.bf16_to_f64(a), datagen.bf16_to_f64(b)
    t0 = time.perf_counter()
    oracle.rel_l1(af, bf)
    t_rl1 = time.perf_counter() - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 exact attention (numpy/BLAS) for {total_rows} query rows of one head "
                   f"at S=118800, D=128 against all keys, {t_attn:.1f} s; rel-L1 over "
                   f"[4096, 3072] bf16 residuals {4 * 4096 * 3072 / t_rl1 / 1e9:.2f} GB/s"),
        "full_step_seconds_extrapolated": 2 * attn_flops(1, 24, S, D) / (tflops * 1e12),
        "int8_oracle": {"quantize_head_s": t_quant, "rows": rows8,
                        "tops": 4.0 * rows8 * S * D / t_int8 / 1e12},
        "cpu_model": cpu_model, "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def time_image_shape(torch, dta, stream, ev, iters=50):
    """bf16 and int8-QK attention at B1 H24 S4608 D128 (a 1024x1024 image DiT), ms per call."""
    B, H, S, D = 1, 24, 4608, 128
    q, k, v = make_inputs(torch, B, H, S, D, seed=1)
    ws = dta.int8qk_workspace(B, H, S, D, "cuda")
    o = torch.empty((B, H, S, D), dtype=torch.float32, device="cuda")
    out = {}
    for name, fn in (("bf16", lambda: dta.attn_fwd_bf16(q, k, v, out=o)),
                     ("int8qk", lambda: dta.attn_fwd_int8qk(q, k, v, out=o, workspace=ws))):
        for _ in range(5):
            fn()
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        # then each call between its own events, for the median
        marks = [ev() for _ in range(iters + 1)]
        marks[0].record(stream)
        for i in range(iters):
            fn()
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        per_call = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(iters))
        out[name] = {"ms": ms, "ms_median": per_call[iters // 2],
                     "tflops": attn_flops(B, H, S, D) / (ms * 1e-3) / 1e12}
    out["bf16"]["frac_bf16_peak"] = out["bf16"]["tflops"] / PEAK_BF16_TFLOPS
    out["int8qk"]["frac_int8_peak"] = out["int8qk"]["tflops"] / PEAK_INT8_TOPS
    out["int8qk"]["frac_mixed_ceiling"] = out["int8qk"]["tflops"] / PEAK_INT8_BF16PV_TOPS
    return out


def time_fbcache(torch, dta, stream, ev, a, b, iters=20):
    """First Block Cache calls on the residual pair: the decision (a rel-L1 pass plus the
    decision, 4 bytes per element) and the residual add (6 bytes per element), GB/s."""
    out_h = torch.empty_like(a)
    st = dta.fbcache_state("cuda")
    cfg = dta.FBCacheConfig()
    ws = torch.empty(dta.rel_l1_workspace_bytes(a.numel()), dtype=torch.uint8, device="cuda")
    res = {}
    for name, fn, nbytes in (
            ("decide", lambda: dta.fbcache_decide(a, b, st, cfg, workspace=ws), 4.0 * a.numel()),
            ("resid_add", lambda: dta.resid_add(a, b, out=out_h), 6.0 * a.numel())):
        for _ in range(3):
            fn()
        e0, e1 = ev(), ev()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": ms, "gbs": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS}
    return res


def time_fp8(torch, dta, stream, ev, q, k, v, o, ws, iters=3, both=False):
    """fp8 attention on the long-video workload (whole call: mean, e4m3 codes, attention);
    both: V in e4m3 too (attn_fwd_fp8), else fp8 QK only (attn_fwd_fp8qk)."""
    if both:
        fn = lambda: dta.attn_fwd_fp8(q, k, v, out=o, workspace=ws)  # noqa: E731
    else:
        fn = lambda: dta.attn_fwd_fp8qk(q, k, v, out=o, workspace=ws)  # noqa: E731
    fn()
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    B, H, S, D = q.shape
    tops = attn_flops(B, H, S, D) / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tops, "frac_fp8_peak": tops / PEAK_INT8_TOPS,
            "note": "whole call; QK and PV on fp8 e4m3 MFMA" if both else
                    "whole call; QK on fp8 e4m3 MFMA, PV bf16"}


def time_extended(torch, dta, stream, ev, q, k, v, iters=2):
    """The extended bf16 call on the long-video workload: q, k, v as [B, S, H, D] views, bf16
    output in that layout and the per-row log-sum-exp (same flops as the plain call)."""
    B, H, S, D = q.shape
    qs, ks, vs = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (q, k, v))
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    fn = lambda: dta.attn_fwd_bf16(qs, ks, vs, out=o, lse=lse)  # noqa: E731
    fn()
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del qs, ks, vs, o, lse
    return {"ms": ms, "tflops": attn_flops(B, H, S, D) / (ms * 1e-3) / 1e12,
            "note": "[B,S,H,D] q/k/v views, bf16 output, lse"}


def time_probe(torch, dta, stream, ev, q, k, v, o_int8, n_rows=256, iters=10):
    """Quantization-error probe on the long-video call: n_rows rows per head, ms per call."""
    B, H, S, D = q.shape
    ws = torch.empty(dta.quant_probe_workspace_bytes(B, H, S, D, n_rows), dtype=torch.uint8,
                     device="cuda")
    err = torch.empty(1 + B * H, dtype=torch.float32, device="cuda")
    fn = lambda: dta.attn_quant_probe(q, k, v, o_int8, n_rows=n_rows, err=err, workspace=ws)  # noqa: E731
    fn()
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return {"ms": e0.elapsed_time(e1) / iters, "rows_per_head": n_rows,
            "err_int8_vs_bf16": float(err[0].item())}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the extra timings (S=4608 attention, First Block Cache calls, "
                         "quantization probe, fp8-QK attention, extended bf16 call): "
                         "profiling runs, one shape per kernel")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the "
                         "reference kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the attention shards by (batch, head) across GPUs, which is not built here)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import diffusion_transformer_attention_amd as dta

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dta.lib()  # fail loudly if the HIP library is missing

    if args.copy_probe:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": src.numel() * 2, "copy_probe_bytes_written": dst.numel() * 2}))
        return

    B, H, S, D = 1, 24, 118800, 128
    RL1_ROWS, RL1_COLS = 118800, 3072
    q, k, v = make_inputs(torch, B, H, S, D, seed=4)
    a, b = make_residuals(torch, RL1_ROWS, RL1_COLS, seed=5)
    o_bf16 = torch.empty((B, H, S, D), dtype=torch.float32, device="cuda")
    o_int8 = torch.empty_like(o_bf16)
    ws8 = dta.int8qk_workspace(B, H, S, D, "cuda")
    r_out = torch.empty(1, dtype=torch.float32, device="cuda")
    ws_rl1 = torch.empty(dta.rel_l1_workspace_bytes(a.numel()), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(marks=None):
        if marks is not None:
            marks[0].record(stream)
        dta.attn_fwd_bf16(q, k, v, out=o_bf16)
        if marks is not None:
            marks[1].record(stream)
        dta.attn_fwd_int8qk(q, k, v, out=o_int8, workspace=ws8)
        if marks is not None:
            marks[2].record(stream)
        dta.resid_rel_l1(a, b, out=r_out, workspace=ws_rl1)
        if marks is not None:
            marks[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    marks = [[ev() for _ in range(4)] for _ in range(args.steps)]
    t_start = ev()
    t_end = ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(marks[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps

    ms_bf16 = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps
    ms_int8 = sum(m[1].elapsed_time(m[2]) for m in marks) / args.steps
    ms_rl1 = sum(m[2].elapsed_time(m[3]) for m in marks) / args.steps
    median = lambda i: sorted(m[i].elapsed_time(m[i + 1]) for m in marks)[args.steps // 2]  # noqa: E731
    F = attn_flops(B, H, S, D)
    value = 2 * F / (ms_step * 1e-3) / 1e12
    bf16_tflops = F / (ms_bf16 * 1e-3) / 1e12
    int8_tops = F / (ms_int8 * 1e-3) / 1e12
    rl1_bytes = 4.0 * a.numel()
    rl1_gbs = rl1_bytes / (ms_rl1 * 1e-3) / 1e9

    # image-DiT shape, timed separately (not part of `value`)
    img = None if args.headline_only else time_image_shape(torch, dta, stream, ev)
    fbc = None if args.headline_only else time_fbcache(torch, dta, stream, ev, a, b)
    probe = None if args.headline_only else time_probe(torch, dta, stream, ev, q, k, v, o_int8)
    fp8 = None if args.headline_only else time_fp8(torch, dta, stream, ev, q, k, v, o_int8, ws8)
    fp8_all = None
    if not args.headline_only:
        ws_f8 = dta.fp8_workspace(B, H, S, D, "cuda")
        fp8_all = time_fp8(torch, dta, stream, ev, q, k, v, o_int8, ws_f8, both=True)
        del ws_f8
    ext = None if args.headline_only else time_extended(torch, dta, stream, ev, q, k, v)

    traffic = load_traffic()
    line = {
        "metric": "DiT attention TFLOP/s + % MFMA peak, bf16 & int8-QK, H=24 D=128, S=4608/118800",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "longvideo attention B1 H24 S118800 D128 (bf16 + int8-QK) "
                               "+ rel-L1 over two bf16 [118800, 3072] residuals",
                   "B": B, "H": H, "S": S, "D": D, "rel_l1_shape": [RL1_ROWS, RL1_COLS],
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": ATTN_KERNEL, "achieved": bf16_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": bf16_tflops / PEAK_BF16_TFLOPS, "traffic": traffic},
        "extra": {
            "bf16": {"ms": ms_bf16, "ms_median": median(0), "tflops": bf16_tflops,
                     "frac_bf16_peak": bf16_tflops / PEAK_BF16_TFLOPS},
            "int8qk": {"ms": ms_int8, "ms_median": median(1), "tops": int8_tops,
                       "frac_int8_peak": int8_tops / PEAK_INT8_TOPS,
                       "frac_mixed_ceiling": int8_tops / PEAK_INT8_BF16PV_TOPS,
                       "note": "whole call: K mean + quantization + attention; the mixed ceiling "
                               "is int8 QK plus bf16 PV at both peaks, 3333 TOPS"},
            "rel_l1": {"ms": ms_rl1, "ms_median": median(2), "gbs": rl1_gbs,
                       "frac_hbm_peak": rl1_gbs / PEAK_HBM_GBS},
            "image_S4608": img,
            "fbcache_118800x3072": fbc,
            "quant_probe": probe,
            "fp8qk": fp8,
            "fp8_qk_pv": fp8_all,
            "bf16_ex_bshd_bf16out_lse": ext,
            "wall_s_timed": wall,
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
