"""GPU: the split of the last round of query tiles (attn_fwd_bf16_ws, and the 8-bit calls, whose
workspace carries the same tail area), against the fp64 oracle and against itself.

When B * H * ceil(S / 256) query tiles are not a multiple of the CU count, the library cuts the
last round's tiles along the key axis into equal ranges, one per CU, and merges each tile's
partial results in key order (csrc/split_plan.h).  Checked here:

* parity with the oracle on every row of shapes whose tail tiles have three or four parts and
  whose workgroups hold two segments (ragged key and query lengths, D = 64 and 128), on the
  bf16, int8-QK and fp8-QK paths, with the tolerances of test_gpu_parity.py, and of fp8 for
  both products against the error model and ceiling of test_gpu_fp8.py;
* strided views, bf16 output and the log-sum-exp through the split;
* the result does not depend on which part arrives last: repeated calls are bit-identical,
  also from a workspace filled with garbage, and the arrival counters are left at zero;
* the split and the whole-tile call agree to bf16 rounding (the parts form their weights at
  their own running offsets, so individual weights round differently).
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
INT8_RELL2 = 1e-2


def announce(msg):
    print(f"[gpu-split] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64(bits):
    return datagen.bf16_to_f64(bits)


def rel_l2(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


def tail_plan(B, H, S):
    """(whole tiles, tail tiles, key tiles) as csrc/split_plan.h plans them on this GPU."""
    G = min(torch.cuda.get_device_properties(0).multi_processor_count, 256)
    n_tiles = B * H * -(-S // 256)
    nkt = -(-S // 64)
    n_main = n_tiles // G * G
    n_tail = n_tiles - n_main
    if n_tail == 0 or n_tail * nkt < 8 * G or 8 * n_tail > 5 * G:
        return n_tiles, 0, nkt
    return n_main, n_tail, nkt


def inputs(B, H, S, D, seed):
    q = datagen.normal_bf16((B, H, S, D), seed, 0)
    k = datagen.f64_to_bf16_bits(f64(datagen.normal_bf16((B, H, S, D), seed, 1)) + 0.75)
    v = datagen.normal_bf16((B, H, S, D), seed, 2)
    return q, k, v


# On 256 workgroups: B1 H5 S4000, 80 tiles of 63 key tiles, about 20 key tiles per workgroup
# (tiles of four parts); B2 H3 S3333, 84 tiles of 53 key tiles, about 17 per workgroup (three
# or four parts).
SHAPES = [(1, 5, 4000, 64), (1, 5, 4000, 128), (2, 3, 3333, 128)]


@pytest.mark.parametrize("B,H,S,D", SHAPES)
def test_split_bf16_every_row(B, H, S, D):
    n_main, n_tail, nkt = tail_plan(B, H, S)
    announce(f"attn_fwd_bf16_ws B{B} H{H} S{S} D{D}: {n_main} whole tiles, {n_tail} split")
    assert n_tail > 0
    q, k, v = inputs(B, H, S, D, 900 + D)
    got = dta.attn_fwd_bf16(dev(q), dev(k), dev(v)).cpu().numpy()
    ref = oracle.attention(f64(q), f64(k), f64(v))
    err, r = np.abs(got - ref).max(), rel_l2(got, ref)
    announce(f"  max-abs {err:.3e} rel-L2 {r:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= BF16_MAXABS and r <= BF16_RELL2, (err, r)


@pytest.mark.parametrize("B,H,S,D", SHAPES[:2])
@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_split_8bit_every_row(B, H, S, D, kind):
    n_main, n_tail, nkt = tail_plan(B, H, S)
    announce(f"attn_fwd_{kind}qk B{B} H{H} S{S} D{D}: {n_tail} split tiles")
    assert n_tail > 0
    q, k, v = inputs(B, H, S, D, 950 + D)
    ws = dta.int8qk_workspace(B, H, S, D, "cuda")
    fn = dta.attn_fwd_int8qk if kind == "int8" else dta.attn_fwd_fp8qk
    got = fn(dev(q), dev(k), dev(v), workspace=ws).cpu().numpy()
    if kind == "int8":
        ref = oracle.quantize_qk(f64(q), f64(k))
        oq = oracle.attention_int8(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], f64(v))
    else:
        ref = oracle.quantize_qk_fp8(f64(q), f64(k))
        oq = oracle.attention_fp8(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], f64(v))
    r = rel_l2(got, oq)
    announce(f"  rel-L2 vs the oracle on the same codes {r:.3e}")
    assert np.all(np.isfinite(got))
    assert r <= INT8_RELL2, r


def lse_tol(S):
    """|lse error| bound (as test_gpu_extended.py): 2^-8 for the bf16 rounding of the weights
    that enter the row sum, S 2^-24 for its fp32 accumulation, 1e-4 for exp2 / log2 and the
    rounding of m + log l."""
    return 2.0 ** -8 + S * 2.0 ** -24 + 1e-4


def test_split_strided_bf16_out_lse():
    B, H, S, D = 1, 5, 4000, 128
    announce(f"attn_fwd_bf16_ws [B, S, H, D] views, bf16 out, lse B{B} H{H} S{S} D{D}")
    q, k, v = inputs(B, H, S, D, 990)
    cq, ck, cv = dev(q), dev(k), dev(v)
    # interleaved heads: [B, S, H, D] storage seen as [B, H, S, D]
    tq, tk, tv = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (cq, ck, cv))
    ref32, lse = dta.attn_fwd_bf16(cq, ck, cv, lse=True)
    ob, lse2 = dta.attn_fwd_bf16(tq, tk, tv, out_dtype=torch.bfloat16, lse=True)
    torch.cuda.synchronize()
    # same plan, same arithmetic: the strided call and the bf16 output are exact
    assert torch.equal(lse, lse2)
    assert torch.equal(ob.contiguous().view(torch.int16), ref32.to(torch.bfloat16).view(torch.int16))
    got = ref32.cpu().numpy()
    ref = oracle.attention(f64(q), f64(k), f64(v))
    err, r = np.abs(got - ref).max(), rel_l2(got, ref)
    lerr = np.abs(lse.cpu().numpy() - oracle.log_sum_exp(f64(q), f64(k))).max()
    announce(f"  max-abs {err:.3e} rel-L2 {r:.3e}; lse max-abs {lerr:.3e} (bound {lse_tol(S):.3e})")
    assert err <= BF16_MAXABS and r <= BF16_RELL2, (err, r)
    assert lerr <= lse_tol(S), lerr


def test_split_deterministic_from_garbage_workspace():
    B, H, S, D = 2, 24, 4608, 128   # 864 tiles: 3 whole rounds and 96 tiles shared out
    n_main, n_tail, nkt = tail_plan(B, H, S)
    announce(f"attn_fwd_bf16_ws determinism B{B} H{H} S{S} D{D}: {n_tail} split tiles")
    assert n_tail > 0
    q, k, v = (dev(x) for x in inputs(B, H, S, D, 1000))
    ws = dta.bf16_workspace(B, H, S, D, "cuda")
    ws.fill_(0xFF)  # counters and slots start as garbage: the call zeroes what it needs
    a = dta.attn_fwd_bf16(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    counters = ws[:4 * max(n_tail, 1)].view(torch.int32).cpu()
    assert int(counters.abs().sum()) == 0, "arrival counters not left at zero"
    for _ in range(3):
        b = dta.attn_fwd_bf16(q, k, v, workspace=ws)
        assert torch.equal(a, b)
    whole = dta.attn_fwd_bf16(q, k, v, workspace=False)
    r = float((a - whole).norm() / whole.norm())
    announce(f"  repeated calls bit-identical; split vs whole tiles rel-L2 {r:.3e}")
    assert r <= 2e-3, r


def test_split_fp8_both_products():
    """fp8 for both products through the split (D = 128): each part rounds its weights to e4m3
    at its own running offset, so the output is held to the fp8-PV error model and ceiling of
    tests/test_gpu_fp8.py against the oracle, not to the element-wise bar."""
    from test_gpu_fp8 import check_out_model, fp8_pv_error_model
    B, H, S, D = 1, 5, 4000, 128
    n_main, n_tail, nkt = tail_plan(B, H, S)
    announce(f"attn_fwd_fp8 B{B} H{H} S{S} D{D}: {n_tail} split tiles")
    assert n_tail > 0
    q, k, v = inputs(B, H, S, D, 1050)
    ws = dta.fp8_workspace(B, H, S, D, "cuda")
    got = dta.attn_fwd_fp8(dev(q), dev(k), dev(v), workspace=ws).cpu().numpy()
    ref = oracle.quantize_qk_fp8(f64(q), f64(k))
    vc, vs = oracle.quantize_v_fp8(f64(v))
    oq = oracle.attention_fp8_full(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], vc, vs)
    vq = oracle.e4m3_value(vc) * vs[:, :, None, :]
    check_out_model(got, oq, oracle.attention(f64(q), f64(k), f64(v)), fp8_pv_error_model(ref, vq),
                    "fp8 QK and PV, split")
