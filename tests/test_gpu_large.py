"""GPU tests at sizes beyond 2^31 elements (64-bit addressing of every tensor).

The long-video workload fits under 2^31 elements per tensor (B1 H24 S118800 D128 = 365M); a
batch of six of them does not (2.19G elements, 4.4 GB per bf16 tensor, 8.8 GB of fp32 output).
Inputs are drawn on the GPU with torch's seeded generator (the distributions of the long-video
workload); only the heads that are checked come back to the host.

  attention   sampled rows of heads at the start, the middle and the end of the batch
              (including the rows whose elements lie beyond 2^31) against exact attention at
              the bf16 bar; the int8 call's K mean, scales and codes of the last head bit-exact
              against the oracle's quantizer on that head, its output on those rows within
              rel-L2 1e-2 of the oracle's int8 attention
  rel-L1      n = 2^31 + 2^20 + 7 elements: b = 1 everywhere, a = b but for a few elements
              (some beyond 2^31, the last one included) that differ by known amounts, so
              sum|a - b| / sum|b| is known exactly; within relative 1e-4
  residuals   resid_add / resid_sub on the same tensors: the elements around the planted ones
              and the tail, bit-exact against the oracle
"""
import math
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
INT8_RELL2 = 1e-2


def announce(msg):
    print(f"[gpu-large] {msg}", file=sys.stderr, flush=True)


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


def test_attention_beyond_2_31_elements():
    B, H, S, D = 6, 24, 118800, 128
    assert B * H * S * D > 2 ** 31
    announce(f"attn_fwd_bf16 / attn_fwd_int8qk B{B} H{H} S{S} D{D} ({B * H * S * D / 2 ** 31:.2f} x 2^31 elements)")
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    shape = (B, H, S, D)
    q = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    off = math.sqrt(2.0) * torch.randn((1, H, 1, D), generator=g, device="cuda")
    k = (torch.randn(shape, generator=g, device="cuda") + off).to(torch.bfloat16)
    v = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
    o = dta.attn_fwd_bf16(q, k, v)
    torch.cuda.synchronize()
    rows = datagen.sample_rows(S, 64, seed=77, edge=32)
    heads = [(0, 0), (3, 11), (B - 1, H - 1)]
    for b, h in heads:
        qh, kh, vh = (host_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
        exact = oracle.attention_rows(qh, kh, vh, rows)
        got = o[b:b + 1, h:h + 1].index_select(2, torch.from_numpy(rows).cuda()).cpu().numpy()
        err, r = np.abs(got - exact).max(), rel_l2(got, exact)
        announce(f"  bf16 (b={b}, h={h}): max-abs {err:.3e} rel-L2 {r:.3e}")
        assert np.all(np.isfinite(got)) and err <= BF16_MAXABS and r <= BF16_RELL2
    del o
    torch.cuda.empty_cache()

    ws = dta.int8qk_workspace(B, H, S, D, "cuda")
    o8 = dta.attn_fwd_int8qk(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    views = dta.int8qk_views(ws, B, H, S, D)
    b, h = B - 1, H - 1
    qh, kh, vh = (host_f64(t[b:b + 1, h:h + 1]) for t in (q, k, v))
    ref = oracle.quantize_qk(qh, kh)
    for key, rk in (("k_mean", "k_mean"), ("q_scale", "q_scale"), ("k_scale", "k_scale"),
                    ("q_codes", "q_codes"), ("k_codes", "k_codes")):
        got = views[key][b:b + 1, h:h + 1].cpu().numpy()
        want = ref[rk]
        same = np.array_equal(got.view(np.uint32), want.view(np.uint32)) if got.dtype == np.float32 \
            else np.array_equal(got, want)
        assert same, f"int8 {key} of head ({b}, {h}) differs from the oracle"
    announce(f"  int8 (b={b}, h={h}): K mean, scales and codes bit-exact")
    oq = oracle.attention_int8(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], vh, rows=rows)
    got = o8[b:b + 1, h:h + 1].index_select(2, torch.from_numpy(rows).cuda()).cpu().numpy()
    r = rel_l2(got, oq)
    announce(f"  int8 (b={b}, h={h}): rel-L2 vs quantized oracle {r:.3e}")
    assert np.all(np.isfinite(got)) and r <= INT8_RELL2
    del q, k, v, o8, ws, views
    torch.cuda.empty_cache()


def test_rel_l1_and_residuals_beyond_2_31_elements():
    n = 2 ** 31 + 2 ** 20 + 7
    announce(f"resid_rel_l1 / resid_add / resid_sub n = 2^31 + 2^20 + 7")
    b = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    a = b.clone()
    # planted differences (all exact in bf16: 1 + delta), some beyond 2^31, the last element too
    idx = np.array([0, 12345, 2 ** 31 - 1, 2 ** 31, 2 ** 31 + 5, n - 8, n - 1], dtype=np.int64)
    delta = np.array([0.5, -0.25, 2.0, -0.5, 0.125, 4.0, -0.75])
    a[torch.from_numpy(idx).cuda()] = torch.from_numpy(1.0 + delta).to(torch.bfloat16).cuda()
    want = float(np.abs(delta).sum()) / n
    got = float(dta.resid_rel_l1(a, b).item())
    announce(f"  rel-L1 {got:.9e}, exact {want:.9e}")
    assert abs(got - want) <= 1e-4 * want
    # residual add / subtract around the planted elements and at the tail
    s, d = dta.resid_add(a, b), dta.resid_sub(a, b)
    torch.cuda.synchronize()
    near = np.unique(np.clip(np.concatenate([idx + o for o in range(-3, 4)]), 0, n - 1))
    ti = torch.from_numpy(near).cuda()
    ab = a.index_select(0, ti).cpu().view(torch.int16).numpy().view(np.uint16)
    bb = b.index_select(0, ti).cpu().view(torch.int16).numpy().view(np.uint16)
    sb = s.index_select(0, ti).cpu().view(torch.int16).numpy().view(np.uint16)
    db = d.index_select(0, ti).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(sb, oracle.resid_add(ab, bb))
    assert np.array_equal(db, oracle.resid_sub(ab, bb))
    announce(f"  resid_add / resid_sub bit-exact at {near.size} elements around the planted ones")
    del a, b, s, d
    torch.cuda.empty_cache()
