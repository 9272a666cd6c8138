"""GPU tests of the quantization-error probe (attn_quant_probe).

What is compared, and the bar:
  chunk results   the probe's bf16 partial outputs for the sampled rows (read from its
                  workspace), merged on the host through their log-sum-exps, against exact
                  attention on those rows: the bf16 path's bar (max-abs <= 2e-2, rel-L2 <= 5e-3)
  the error       err[0] and err[1 + bh] against the same relative L2 recomputed on the host
                  from those merged rows and the quantized call's output: within 1e-5 relative
                  (only the fp64 summation order differs)
  vs the oracle   against oracle.quant_probe_error (int8 attention on the oracle's codes vs
                  exact attention), within the triangle-inequality bound
                  (|o8 - o8*| + |o - o*|) / |o| * (1 + err*) + 1e-6, both distances measured
"""
import sys

import numpy as np
import pytest

import datagen
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import diffusion_transformer_attention_amd as dta  # noqa: E402

BF16_MAXABS, BF16_RELL2 = 2e-2, 5e-3


def announce(msg):
    print(f"[gpu-probe] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64(bits):
    return datagen.bf16_to_f64(bits)


def merged_rows(views):
    n = len(views["chunks"])
    part = views["part"][:, :n].cpu().numpy().astype(np.float64)   # [B, n, H, R, D]
    lse = views["lse"][:, :n].cpu().numpy().astype(np.float64)
    m = lse.max(axis=1, keepdims=True)
    w = np.exp(lse - m)
    return (w[..., None] * part).sum(axis=1) / w.sum(axis=1)[..., None]


def rel_l2(x, y, axis=None):
    return np.sqrt(((x - y) ** 2).sum(axis=axis) / (y ** 2).sum(axis=axis))


def run_probe(q, k, v, n_rows, o8_bf16=False, layout="bhsd"):
    B, H, S, D = q.shape
    qd, kd, vd = dev(q), dev(k), dev(v)
    if layout == "bshd":
        qd, kd, vd = (t.permute(0, 2, 1, 3).contiguous().transpose(1, 2) for t in (qd, kd, vd))
    o8 = dta.attn_fwd_int8qk(qd, kd, vd, out_dtype=torch.bfloat16 if o8_bf16 else None)
    ws = torch.empty(dta.quant_probe_workspace_bytes(B, H, S, D, n_rows), dtype=torch.uint8,
                     device="cuda")
    err = dta.attn_quant_probe(qd, kd, vd, o8, n_rows=n_rows, workspace=ws)
    torch.cuda.synchronize()
    views = dta.quant_probe_views(ws, B, H, S, D, n_rows)
    rows = oracle.probe_rows(S, n_rows)
    o8_rows = o8.float().cpu().numpy()[:, :, rows].astype(np.float64)
    return err.cpu().numpy(), merged_rows(views), o8_rows, len(views["chunks"])


CASES = [
    # B, H, S, D, n_rows, layout, bf16 o_q
    (1, 2, 1000, 64, 100, "bhsd", False),
    (1, 3, 4608, 128, 256, "bhsd", False),
    (2, 2, 3000, 128, 77, "bshd", True),
    (1, 2, 130, 64, 130, "bhsd", False),
]


@pytest.mark.parametrize("B,H,S,D,R,layout,o8_bf16", CASES)
def test_probe_against_host_and_oracle(B, H, S, D, R, layout, o8_bf16):
    announce(f"attn_quant_probe B{B} H{H} S{S} D{D} rows {R} {layout} o_q {'bf16' if o8_bf16 else 'fp32'}")
    q = datagen.normal_bf16((B, H, S, D), 900 + S, 0)
    k = datagen.f64_to_bf16_bits(f64(datagen.normal_bf16((B, H, S, D), 900 + S, 1)) + 1.0)
    v = datagen.normal_bf16((B, H, S, D), 900 + S, 2)
    err, o16, o8, ns = run_probe(q, k, v, R, o8_bf16, layout)
    rows = oracle.probe_rows(S, R)
    exact = oracle.attention_rows(f64(q), f64(k), f64(v), rows)
    # the probe's bf16 rows: the bf16 path's bar against exact attention
    mx, r2 = np.abs(o16 - exact).max(), rel_l2(o16, exact)
    announce(f"  {ns} key chunks; merged rows vs exact: max-abs {mx:.2e} rel-L2 {r2:.2e}")
    assert mx <= BF16_MAXABS and r2 <= BF16_RELL2
    # the error values: the host's relative L2 on the same rows
    host_head = rel_l2(o8, o16, axis=(2, 3))
    host_all = rel_l2(o8, o16)
    np.testing.assert_allclose(err[1:], host_head.ravel(), rtol=1e-5, atol=1e-7)
    assert abs(err[0] - host_all) <= 1e-5 * host_all + 1e-7
    # against the oracle's error
    o_all, o_head = oracle.quant_probe_error(f64(q), f64(k), f64(v), R)
    qq = oracle.quantize_qk(f64(q), f64(k))
    o8_ref = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"],
                                   f64(v), rows=rows)
    n16 = np.sqrt((o16 ** 2).sum())
    bound = (np.sqrt(((o8 - o8_ref) ** 2).sum()) + np.sqrt(((o16 - exact) ** 2).sum())) / n16
    bound = bound * (1 + o_all) + 1e-6
    announce(f"  err {err[0]:.4e}, oracle {o_all:.4e}, bound {bound:.2e}")
    assert abs(err[0] - o_all) <= bound
    assert 1e-3 < err[0] < 0.1


def test_probe_longvideo_shape():
    """The long-video shape with 256 rows per head: ten chunks of 11840 keys and a tail."""
    B, H, S, D, R = 1, 24, 118800, 128, 256
    announce(f"attn_quant_probe longvideo B{B} H{H} S{S} D{D} rows {R}")
    q, k, v = datagen.attention_inputs("longvideo")
    qd, kd, vd = dev(q), dev(k), dev(v)
    o8 = dta.attn_fwd_int8qk(qd, kd, vd)
    ws = torch.empty(dta.quant_probe_workspace_bytes(B, H, S, D, R), dtype=torch.uint8, device="cuda")
    err = dta.attn_quant_probe(qd, kd, vd, o8, n_rows=R, workspace=ws)
    torch.cuda.synchronize()
    views = dta.quant_probe_views(ws, B, H, S, D, R)
    assert len(views["chunks"]) == 11      # ten chunks of 11840 keys and a tail of 400
    rows = oracle.probe_rows(S, R)
    o16 = merged_rows(views)
    o8_rows = o8.cpu().numpy()[:, :, rows].astype(np.float64)
    del qd, kd, vd, o8, ws
    torch.cuda.empty_cache()
    e = err.cpu().numpy()
    np.testing.assert_allclose(e[1:], rel_l2(o8_rows, o16, axis=(2, 3)).ravel(), rtol=1e-5, atol=1e-7)
    # exact attention on a few of the sampled rows of two heads
    pick = np.array([0, 100, 255])
    for h in (0, 23):
        ex = oracle.attention_rows(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]), rows[pick])
        got = o16[:, h:h + 1][:, :, pick]
        assert np.abs(got - ex).max() <= BF16_MAXABS and rel_l2(got, ex) <= BF16_RELL2
    announce(f"  err {e[0]:.4e} (per head {e[1:].min():.3e} .. {e[1:].max():.3e})")
    assert 1e-3 < e[0] < 0.1
