"""GPU: long calls with bf16 V read V through V^T tiles (S >= 32768 at D = 128, with a
workspace): bf16, int8-QK and fp8-QK attention.

The tiles are written by a prepass (64 keys of 128 channels each, every 16-key step in the key
order of the weights operand), and the attention reads each PV operand with one 16-byte LDS
read instead of two transposing ones.  The products see the same values in the same order, so:

* where a call has no shared-out last round (B1 H2 S33000: 258 tiles, the last round too short
  to split), the workspace call through the tiles is bit-identical to the plain call, which
  reads V as it is; both are also checked against the fp64 oracle on every row;
* a strided V (interleaved heads) gives the same tiles and the same output bits as the
  contiguous one and as the plain call, with one batch of two heads and with two batches of one
  head;
* the bf16 output and the log-sum-exp through the tiles are bit-identical to the plain call's;
* with a shared-out last round (B1 H24 S33000) the output is checked against the oracle on
  sampled rows of every head, at the bars of test_gpu_parity.py, and repeated calls from a
  garbage workspace are bit-identical;
* the int8-QK and fp8-QK calls (always on a workspace) are checked on sampled rows against the
  oracle's attention on the same codes, and their codes bit-exact, as in test_gpu_parity.py and
  test_gpu_fp8.py.
The ragged length (33000 = 515 * 64 + 40) puts the last key tile on the final 64 rows, as the
K tile, with the keys it shares with the previous tile masked.
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
S_LONG = 33000


def announce(msg):
    print(f"[gpu-vt] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64(bits):
    return datagen.bf16_to_f64(bits)


def rel_l2(x, y):
    return float(np.linalg.norm((x - y).ravel()) / np.linalg.norm(y.ravel()))


def inputs(B, H, S, D, seed):
    q = datagen.normal_bf16((B, H, S, D), seed, 0)
    k = datagen.f64_to_bf16_bits(f64(datagen.normal_bf16((B, H, S, D), seed, 1)) + 0.5)
    v = datagen.normal_bf16((B, H, S, D), seed, 2)
    return q, k, v


def uses_vt(B, H, S, D):
    """The bf16 workspace holds V^T tiles (64-key tiles of 128 x 64 bf16) beyond the tail area."""
    return dta.bf16_workspace_bytes(B, H, S, D) >= B * H * -(-S // 64) * 128 * 64 * 2


def test_vt_bf16_bit_identical_and_every_row():
    B, H, S, D = 1, 2, S_LONG, 128
    assert uses_vt(B, H, S, D)
    announce(f"bf16 B{B} H{H} S{S} D{D}: V^T tiles (workspace) vs V as it is (plain call)")
    q, k, v = inputs(B, H, S, D, 1200)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = dta.bf16_workspace(B, H, S, D, "cuda")
    ws.fill_(0xFF)
    a = dta.attn_fwd_bf16(qd, kd, vd, workspace=ws)
    b = dta.attn_fwd_bf16(qd, kd, vd, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "V^T tiles change the output"
    got = a.cpu().numpy()
    ref = oracle.attention(f64(q), f64(k), f64(v))
    err, r = np.abs(got - ref).max(), rel_l2(got, ref)
    announce(f"  bit-identical; every row: max-abs {err:.3e} rel-L2 {r:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= BF16_MAXABS and r <= BF16_RELL2, (err, r)


@pytest.mark.parametrize("B,H", [(1, 2), (2, 1)])
def test_vt_strided_v_same_bits(B, H):
    S, D = S_LONG, 128
    announce(f"bf16 B{B} H{H} S{S} D{D}: [B, S, H, D] views through V^T tiles")
    q, k, v = (dev(x) for x in inputs(B, H, S, D, 1210))
    ref = dta.attn_fwd_bf16(q, k, v)
    plain = dta.attn_fwd_bf16(q, k, v, workspace=False)  # V as it is (258 tiles: no split either)
    tq, tk, tv = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    got = dta.attn_fwd_bf16(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(ref, plain)
    announce("  bit-identical to the contiguous call and to the call that reads V as it is")


def test_vt_bf16_output_and_lse_same_bits():
    """bf16 output and the per-row log-sum-exp through the V^T tiles: bit-identical to the plain
    call (B1 H2 S33000 has no shared-out round)."""
    B, H, S, D = 1, 2, S_LONG, 128
    announce(f"bf16 B{B} H{H} S{S} D{D}: bf16 output and lse through V^T tiles")
    q, k, v = (dev(x) for x in inputs(B, H, S, D, 1215))
    o1, l1 = dta.attn_fwd_bf16(q, k, v, out_dtype=torch.bfloat16, lse=True)
    o2, l2 = dta.attn_fwd_bf16(q, k, v, out_dtype=torch.bfloat16, lse=True, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    announce("  bf16 output and lse bit-identical to the plain call")


def test_vt_with_shared_out_round_sampled():
    """B1 H24 S33000: 3096 tiles, 12 whole rounds and 24 tiles shared out over the CUs, through
    V^T tiles; sampled rows of every head against the oracle, and repeated calls from a
    garbage workspace bit-identical."""
    B, H, S, D = 1, 24, S_LONG, 128
    assert uses_vt(B, H, S, D)
    announce(f"bf16 B{B} H{H} S{S} D{D}: V^T tiles and a shared-out last round")
    q, k, v = inputs(B, H, S, D, 1220)
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws = dta.bf16_workspace(B, H, S, D, "cuda")
    ws.fill_(0xFF)
    a = dta.attn_fwd_bf16(qd, kd, vd, workspace=ws)
    c = dta.attn_fwd_bf16(qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
    rows = datagen.sample_rows(S, 64, seed=78)
    got = a.index_select(2, torch.from_numpy(rows).cuda()).cpu().numpy()
    ref = np.empty_like(got, dtype=np.float64)
    for h in range(H):
        sl = (slice(0, 1), slice(h, h + 1))
        ref[sl] = oracle.attention_rows(f64(q[sl]), f64(k[sl]), f64(v[sl]), rows)
    err, r = np.abs(got - ref).max(), rel_l2(got, ref)
    announce(f"  {rows.size} rows per head: max-abs {err:.3e} rel-L2 {r:.3e}")
    assert err <= BF16_MAXABS and r <= BF16_RELL2, (err, r)


@pytest.mark.parametrize("kind", ["int8", "fp8"])
def test_vt_8bit_sampled(kind):
    B, H, S, D = 1, 2, S_LONG, 128
    announce(f"attn_fwd_{kind}qk B{B} H{H} S{S} D{D} through V^T tiles")
    q, k, v = inputs(B, H, S, D, 1230)
    ws = dta.int8qk_workspace(B, H, S, D, "cuda")
    ws.fill_(0xFF)
    fn = dta.attn_fwd_int8qk if kind == "int8" else dta.attn_fwd_fp8qk
    out = fn(dev(q), dev(k), dev(v), workspace=ws)
    torch.cuda.synchronize()
    views = {n: t.cpu().numpy() for n, t in dta.int8qk_views(ws, B, H, S, D).items()}
    if kind == "fp8":  # e4m3 bytes
        for n in ("q_codes", "k_codes"):
            views[n] = views[n].view(np.uint8)
    rows = datagen.sample_rows(S, 256, seed=79)
    got = out.index_select(2, torch.from_numpy(rows).cuda()).cpu().numpy()
    ref = (oracle.quantize_qk if kind == "int8" else oracle.quantize_qk_fp8)(f64(q), f64(k))
    for key in ("q_codes", "k_codes"):
        assert int(np.sum(views[key] != ref[key])) == 0, key
    for key in ("k_mean", "q_scale", "k_scale"):
        assert int(np.sum(views[key].view(np.uint32) != ref[key].view(np.uint32))) == 0, key
    attend = oracle.attention_int8 if kind == "int8" else oracle.attention_fp8
    oq = attend(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], f64(v), rows=rows)
    r = rel_l2(got, oq)
    announce(f"  codes bit-exact; {rows.size} rows per head: rel-L2 vs the oracle on the same codes {r:.3e}")
    assert np.all(np.isfinite(got))
    assert r <= INT8_RELL2, r
