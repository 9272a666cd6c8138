"""GPU tests of the extended attention calls (attn_fwd_bf16_ex, attn_fwd_int8qk_ex): strided
views, bf16 output and the per-row log-sum-exp.

What is compared, and the bar:
  strided views    bit-identical to the plain call on contiguous copies (same arithmetic,
                   only the addresses differ); int8: identical codes, scales and K mean too
  bf16 output      bit-identical to the fp32 output rounded to nearest even
  lse              against the oracle's log-sum-exp (exact scores, or the int8 path's
                   quantized scores on the call's own codes), |error| <= LSE_TOL(S) with
                     2^-8       every weight that enters the row sum is rounded to bf16
                                (relative error <= 2^-8, so the log of the sum moves <= 2^-8)
                     S * 2^-24  fp32 accumulation of S positive terms
                     1e-4       v_exp_f32 / v_log_f32 approximation and fp32 rounding of m + log l
                   plus, for the int8 path, the rounding of the bias correction
                   (0.75 * q_scale * k_scale * scale, see test_int8_lse_vs_oracle)
  split keys       two calls over disjoint key sets merged through their lse against exact
                   attention over all keys, at the bf16 path's tolerance
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


def lse_tol(S):
    return 2.0 ** -8 + S * 2.0 ** -24 + 1e-4


def announce(msg):
    print(f"[gpu-extended] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64(bits):
    return datagen.bf16_to_f64(bits)


def inputs(B, H, S, D, seed):
    return tuple(datagen.normal_bf16((B, H, S, D), seed, t) for t in range(3))


def rel_l2(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


def bshd_view(t):
    """The same values as [B, H, S, D] t, stored [B, S, H, D], viewed as [B, H, S, D]."""
    return t.permute(0, 2, 1, 3).contiguous().transpose(1, 2)


def fused_qkv_views(q, k, v):
    """q, k, v as slices of one [B, S, 3, H, D] projection output (token stride 3 H D)."""
    qkv = torch.stack([t.permute(0, 2, 1, 3) for t in (q, k, v)], dim=2).contiguous()
    return tuple(qkv[:, :, i].transpose(1, 2) for i in range(3))


def sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------------
# strided views and output dtype: same bits as the plain call
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("S,D", [(65, 64), (300, 128), (1000, 64), (4608, 128)])
def test_bf16_strided_views_bit_identical(S, D):
    B, H = 2, 3
    announce(f"attn_fwd_bf16_ex strided views B{B} H{H} S{S} D{D}")
    q, k, v = (dev(x) for x in inputs(B, H, S, D, 700 + D))
    ref = dta.attn_fwd_bf16(q, k, v)
    # [B, S, H, D] storage; the output follows q's layout
    qs, ks, vs = bshd_view(q), bshd_view(k), bshd_view(v)
    o1 = dta.attn_fwd_bf16(qs, ks, vs)
    assert o1.stride(1) < o1.stride(2)
    # fused QKV, output into a padded buffer
    qf, kf, vf = fused_qkv_views(q, k, v)
    pad = torch.full((B, H, S + 5, D), float("nan"), device="cuda")
    o2 = dta.attn_fwd_bf16(qf, kf, vf, out=pad[:, :, :S])
    # K and V shared by all heads (head stride 0), against the same values made contiguous
    k1, v1 = k[:, :1].expand(B, H, S, D), v[:, :1].expand(B, H, S, D)
    o3 = dta.attn_fwd_bf16(q, k1, v1, lse=True)[0]
    ref3 = dta.attn_fwd_bf16(q, k1.contiguous(), v1.contiguous())
    sync()
    assert torch.equal(o1, ref), "[B, S, H, D] layout"
    assert torch.equal(o2, ref), "fused QKV"
    assert torch.isnan(pad[:, :, S:]).all(), "wrote outside the output view"
    assert torch.equal(o3, ref3), "broadcast K/V"


@pytest.mark.parametrize("S,D", [(129, 128), (1000, 64)])
def test_bf16_output_is_rounded_fp32(S, D):
    announce(f"attn_fwd_bf16_ex bf16 output B1 H2 S{S} D{D}")
    q, k, v = (dev(x) for x in inputs(1, 2, S, D, 710 + D))
    ref = dta.attn_fwd_bf16(q, k, v)
    ob = dta.attn_fwd_bf16(q, k, v, out_dtype=torch.bfloat16)
    ob2 = dta.attn_fwd_bf16(bshd_view(q), bshd_view(k), bshd_view(v), out_dtype=torch.bfloat16)
    sync()
    assert ob.dtype == torch.bfloat16
    expect = ref.to(torch.bfloat16)  # round to nearest even
    assert torch.equal(ob.view(torch.int16), expect.view(torch.int16))
    assert torch.equal(ob2.contiguous().view(torch.int16), expect.view(torch.int16))


@pytest.mark.parametrize("S,D", [(63, 128), (300, 64), (4608, 128)])
def test_int8_strided_views_bit_identical(S, D):
    B, H = 1, 3
    announce(f"attn_fwd_int8qk_ex strided views B{B} H{H} S{S} D{D}")
    q, k, v = (dev(x) for x in inputs(B, H, S, D, 720 + D))
    k = (k.float() + 0.75).bfloat16()  # a channel offset for the mean to remove
    ws0 = dta.int8qk_workspace(B, H, S, D, "cuda")
    ws1 = dta.int8qk_workspace(B, H, S, D, "cuda")
    ref = dta.attn_fwd_int8qk(q, k, v, workspace=ws0)
    qf, kf, vf = fused_qkv_views(q, k, v)
    o1, lse = dta.attn_fwd_int8qk(qf, kf, vf, workspace=ws1, lse=True)
    ob = dta.attn_fwd_int8qk(bshd_view(q), bshd_view(k), bshd_view(v), out_dtype=torch.bfloat16)
    sync()
    v0 = dta.int8qk_views(ws0, B, H, S, D)
    v1 = dta.int8qk_views(ws1, B, H, S, D)
    for name in v0:
        assert torch.equal(v0[name], v1[name]), name
    assert torch.equal(o1.contiguous(), ref)
    assert torch.equal(ob.contiguous().view(torch.int16), ref.to(torch.bfloat16).view(torch.int16))
    assert torch.isfinite(lse).all()


# ---------------------------------------------------------------------------------------------
# log-sum-exp against the oracle
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("S,D", [(1, 64), (65, 128), (300, 64), (1000, 128)])
def test_bf16_lse_vs_oracle(S, D):
    announce(f"attn_fwd_bf16_ex lse B2 H2 S{S} D{D}")
    qb, kb, vb = inputs(2, 2, S, D, 730 + D)
    q, k, v = dev(qb), dev(kb), dev(vb)
    o, lse = dta.attn_fwd_bf16(q, k, v, lse=True)
    ref_o = dta.attn_fwd_bf16(q, k, v)
    sync()
    assert torch.equal(o, ref_o), "asking for lse changed the output"
    ref = oracle.log_sum_exp(f64(qb), f64(kb))
    err = np.abs(lse.cpu().numpy() - ref).max()
    announce(f"S={S} D={D}: lse max error {err:.3e} (bound {lse_tol(S):.3e})")
    assert err <= lse_tol(S)


def test_bf16_lse_large_scores():
    """Scores near a hundred (softmax nearly one-hot, lse close to the largest score)."""
    S, D = 500, 128
    announce(f"attn_fwd_bf16_ex lse with large scores B1 H2 S{S} D{D}")
    qb, kb, vb = inputs(1, 2, S, D, 740)
    qb = datagen.f64_to_bf16_bits(f64(qb) * 6.0)
    kb = datagen.f64_to_bf16_bits(f64(kb) * 6.0)
    _, lse = dta.attn_fwd_bf16(dev(qb), dev(kb), dev(vb), lse=True)
    sync()
    ref = oracle.log_sum_exp(f64(qb), f64(kb))
    assert ref.max() > 50
    # on top of the bound: fp32 accumulation of the D products of a score, at most
    # D * 2^-24 * sum_d |q_d k_d| * scale <= D * 2^-24 * |q| |k| * scale (Cauchy-Schwarz)
    qn = np.linalg.norm(f64(qb), axis=-1).max()
    kn = np.linalg.norm(f64(kb), axis=-1).max()
    tol = lse_tol(S) + D * 2.0 ** -24 * qn * kn / np.sqrt(D)
    err = np.abs(lse.cpu().numpy() - ref).max()
    announce(f"large scores: lse max error {err:.3e} (bound {tol:.3e})")
    assert err <= tol


def test_bf16_lse_image_sampled():
    announce("attn_fwd_bf16_ex lse image B1 H24 S4608 D128 (sampled rows)")
    q, k, v = datagen.attention_inputs("image")
    S = q.shape[2]
    _, lse = dta.attn_fwd_bf16(dev(q), dev(k), dev(v), lse=True)
    sync()
    rows = datagen.sample_rows(S, 128, seed=78)
    ref = oracle.log_sum_exp(f64(q[:, :, rows]), f64(k))
    err = np.abs(lse.cpu().numpy()[:, :, rows] - ref).max()
    announce(f"image: lse max error {err:.3e} (bound {lse_tol(S):.3e})")
    assert err <= lse_tol(S)


@pytest.mark.parametrize("S,D", [(65, 64), (300, 128), (1000, 64)])
def test_int8_lse_vs_oracle(S, D):
    B, H = 1, 3
    announce(f"attn_fwd_int8qk_ex lse B{B} H{H} S{S} D{D}")
    qb, kb, vb = inputs(B, H, S, D, 750 + D)
    kb = datagen.f64_to_bf16_bits(f64(kb) + 1.5)
    ws = dta.int8qk_workspace(B, H, S, D, "cuda")
    _, lse = dta.attn_fwd_int8qk(dev(qb), dev(kb), dev(vb), workspace=ws, lse=True)
    sync()
    views = {n: t.cpu().numpy() for n, t in dta.int8qk_views(ws, B, H, S, D).items()}
    # the codes themselves are pinned bit-exact to the oracle's quantizer elsewhere
    ref_q = oracle.quantize_qk(f64(qb), f64(kb))
    for name in ("q_codes", "k_codes"):
        assert np.array_equal(views[name], ref_q[name]), name
    ref = oracle.log_sum_exp_int8(views["q_codes"], views["q_scale"], views["k_codes"],
                                  views["k_scale"])
    scale = 1.0 / np.sqrt(D)
    # the kernel carries each tile's integer scores offset by 1.5 * 2^23 and removes the offset
    # with one fp32 product of it and the score factor: its rounding moves a tile's scores by at
    # most 2^-24 * 1.5 * 2^23 * q_scale * k_scale * scale (natural-log units)
    bias_err = 0.75 * views["q_scale"].max() * views["k_scale"].max() * scale
    tol = lse_tol(S) + bias_err
    err = np.abs(lse.cpu().numpy() - ref).max()
    announce(f"int8 S={S} D={D}: lse max error {err:.3e} (bound {tol:.3e})")
    assert err <= tol


# ---------------------------------------------------------------------------------------------
# keys split over two calls, merged through lse
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("S,D", [(300, 64), (1000, 128)])
def test_bf16_split_keys_merge(S, D):
    announce(f"attn_fwd_bf16_ex split keys B1 H2 S{S}+{S} D{D}")
    qb, ka, va = inputs(1, 2, S, D, 760 + D)
    _, kb, vb = inputs(1, 2, S, D, 770 + D)
    q = dev(qb)
    oa, la = dta.attn_fwd_bf16(q, dev(ka), dev(va), lse=True)
    ob, lb = dta.attn_fwd_bf16(q, dev(kb), dev(vb), lse=True)
    sync()
    oa, la, ob, lb = (t.cpu().numpy().astype(np.float64) for t in (oa, la, ob, lb))
    lse = np.logaddexp(la, lb)
    merged = np.exp(la - lse)[..., None] * oa + np.exp(lb - lse)[..., None] * ob
    exact = oracle.attention(f64(qb), np.concatenate([f64(ka), f64(kb)], axis=2),
                             np.concatenate([f64(va), f64(vb)], axis=2))
    err, r = np.abs(merged - exact).max(), rel_l2(merged, exact)
    announce(f"split keys: max-abs {err:.3e} rel-L2 {r:.3e}")
    assert err <= BF16_MAXABS and r <= BF16_RELL2
    ref_lse = oracle.log_sum_exp(f64(qb), np.concatenate([f64(ka), f64(kb)], axis=2))
    assert np.abs(lse - ref_lse).max() <= lse_tol(2 * S)
