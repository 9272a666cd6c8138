"""The C ABI library: it loads, exports every declared entry point, sizes its workspaces as
documented, and rejects bad arguments before touching the GPU (no GPU needed)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ditattn.h")

EINVAL, EUNSUP, EWS = -1, -2, -3
FAKE = 0x100000  # a 256-byte aligned address the library never dereferences on invalid calls


@pytest.fixture(scope="module")
def L():
    import diffusion_transformer_attention_amd as dta
    # DITATTN_ABI_LIB: run these checks on another build of the same sources, e.g. the
    # host-instrumented one of tests/run_abi_asan.py
    alt = os.environ.get("DITATTN_ABI_LIB")
    if alt:
        return dta.declare(ctypes.CDLL(alt))
    if not os.path.exists(dta.LIB_PATH):
        from diffusion_transformer_attention_amd.build import build
        build()
    return dta.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"DITATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("attn_fwd_bf16", "attn_fwd_int8qk", "resid_rel_l1", "attn_fwd_bf16_ex",
              "attn_fwd_int8qk_ex", "fbcache_decide", "resid_add", "resid_sub",
              "attn_quant_probe", "attn_fwd_fp8qk", "attn_fwd_fp8qk_ex", "attn_fwd_fp8",
              "attn_fwd_fp8_ex", "resid_rel_l1_noalloc", "attn_fwd_bf16_ws",
              "attn_bf16_workspace_bytes"):
        assert n in names
    assert len(names) == 25


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert L.ditattn_status_string(s)


def _align(x, a=256):
    return (x + a - 1) // a * a


@pytest.mark.parametrize("B,H,S,D", [(1, 2, 256, 64), (1, 24, 4608, 128), (2, 24, 11440, 128),
                                     (1, 24, 118800, 128), (3, 1, 1, 64)])
def test_int8_workspace_layout(L, B, H, S, D):
    off = (ctypes.c_size_t * 6)()
    total = L.attn_int8qk_workspace_offsets(B, H, S, D, off)
    assert total == L.attn_int8qk_workspace_bytes(B, H, S, D)
    sizes = [B * H * D * 4, B * H * math.ceil(S / 128) * 4, B * H * math.ceil(S / 64) * 4,
             B * H * S * D, B * H * S * D]
    expect = 0
    for i, sz in enumerate(sizes):
        assert off[i] == expect and off[i] % 256 == 0
        expect = _align(expect + sz)
    assert off[5] == expect and total > off[5] and total % 256 == 0
    # the scratch segment also holds the attention's tail workspace and V^T tiles
    assert total - off[5] >= _align(_tail_bytes(S, D)) + _vt_bytes(B, H, S, D)


@pytest.mark.parametrize("B,H,S,D", [(1, 2, 256, 128), (1, 24, 118800, 128), (3, 1, 1, 128)])
def test_fp8_workspace_layout(L, B, H, S, D):
    off6 = (ctypes.c_size_t * 6)()
    base = L.attn_int8qk_workspace_offsets(B, H, S, D, off6)
    off = (ctypes.c_size_t * 9)()
    total = L.attn_fp8_workspace_offsets(B, H, S, D, off)
    assert total == L.attn_fp8_workspace_bytes(B, H, S, D)
    assert list(off)[:6] == list(off6) and off[6] == base
    assert off[7] == _align(off[6] + B * H * D * 4)
    assert off[8] == _align(off[7] + B * H * S * D)
    assert total > off[8] and total % 256 == 0


def test_fp8_all_argument_errors(L):
    need = L.attn_fp8_workspace_bytes(1, 1, 64, 128)
    args = [FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, 1, 1, 64, 128, 0.125]
    assert L.attn_fwd_fp8(*args, None, need, None) == EWS
    assert L.attn_fwd_fp8(*args, FAKE + 0x8000, need - 1, None) == EWS
    bad = list(args); bad[7] = 64                      # fp8 V is laid out for D = 128 only
    assert L.attn_fwd_fp8(*bad, FAKE + 0x8000, 1 << 30, None) == EUNSUP
    bad = list(args); bad[0] = None
    assert L.attn_fwd_fp8(*bad, FAKE + 0x8000, need, None) == EINVAL
    st = (ctypes.c_int64 * 12)(*_contig(1, 64, 128))
    assert L.attn_fwd_fp8_ex(FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, 5, None, st, 1, 1,
                             64, 128, 0.125, FAKE + 0x8000, need, None) == EINVAL


def _tail_bytes(S, D):
    """The split of the last round: 256 counters (1 KB), then 2 slots for each of up to 256
    workgroups, a slot holding 512 lanes x (D/2 O values + m + l) fp32; none for 8 key tiles or
    fewer (ranges of 8 key tiles, each shorter than a tile)."""
    if math.ceil(S / 64) <= 8:
        return 0
    return 1024 + 2 * 256 * 512 * (D // 2 + 2) * 4


def _vt_bytes(B, H, S, D):
    """V^T tiles of long bf16 and int8-QK calls (D = 128, S >= 32768): per (b, h) one tile of
    128 channel rows x 64 bf16 keys per 64-key tile."""
    if D != 128 or S < 32768:
        return 0
    return B * H * math.ceil(S / 64) * 128 * 64 * 2


@pytest.mark.parametrize("S", [1, 64, 448, 449, 512, 4608, 11440, 32767, 32768, 33000, 118800])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_workspace_size(L, S, D):
    want = max(_align(_tail_bytes(S, D)) + _vt_bytes(1, 24, S, D), 256)
    assert L.attn_bf16_workspace_bytes(1, 24, S, D) == want
    assert L.attn_bf16_workspace_bytes(1, 24, S, 96) == 0
    assert L.attn_bf16_workspace_bytes(0, 24, S, D) == 0


def test_bf16_ws_argument_errors(L):
    st = (ctypes.c_int64 * 12)(*_contig(1, 4608, 128))
    need = L.attn_bf16_workspace_bytes(1, 1, 4608, 128)
    args = [FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, 0, None, st, 1, 1, 4608, 128, 0.125]
    assert L.attn_fwd_bf16_ws(*args, None, need, None) == EWS
    assert L.attn_fwd_bf16_ws(*args, FAKE + 0x8000, need - 1, None) == EWS
    assert L.attn_fwd_bf16_ws(*args, FAKE + 0x8010, need, None) == EWS   # not 256-aligned
    bad = list(args); bad[4] = 7                                          # out_dtype
    assert L.attn_fwd_bf16_ws(*bad, FAKE + 0x8000, need, None) == EINVAL
    bad = list(args); bad[6] = None                                       # strides
    assert L.attn_fwd_bf16_ws(*bad, FAKE + 0x8000, need, None) == EINVAL
    bad = list(args); bad[10] = 96
    assert L.attn_fwd_bf16_ws(*bad, FAKE + 0x8000, need, None) == EUNSUP
    bad = list(args); bad[3] = FAKE                                       # o aliases q
    assert L.attn_fwd_bf16_ws(*bad, FAKE + 0x8000, need, None) == EINVAL


def test_invalid_shapes_give_zero_workspace(L):
    assert L.attn_int8qk_workspace_bytes(0, 1, 1, 64) == 0
    assert L.attn_int8qk_workspace_bytes(1, 1, 0, 64) == 0
    assert L.attn_int8qk_workspace_bytes(1, 1, 8, 96) == 0
    assert L.resid_rel_l1_workspace_bytes(0) == 0
    assert L.resid_rel_l1_workspace_bytes(1) >= 16
    assert L.resid_rel_l1_workspace_bytes(364953600) >= 16


def _bf16(L, q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, o=FAKE + 0x3000, B=1, H=1, S=64, D=64,
          scale=0.125):
    return L.attn_fwd_bf16(q, k, v, o, B, H, S, D, scale, None)


def test_bf16_argument_errors(L):
    assert _bf16(L, q=None) == EINVAL
    assert _bf16(L, o=None) == EINVAL
    assert _bf16(L, k=FAKE + 8) == EINVAL             # misaligned
    assert _bf16(L, o=FAKE) == EINVAL                 # output aliases q
    assert _bf16(L, B=0) == EINVAL
    assert _bf16(L, S=-5) == EINVAL
    assert _bf16(L, D=96) == EUNSUP
    assert _bf16(L, D=256) == EUNSUP
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _bf16(L, scale=bad) == EINVAL
    assert _bf16(L, B=1 << 20, H=1 << 10, S=1 << 20) == EINVAL  # grid would overflow


@pytest.mark.parametrize("name", ["attn_fwd_int8qk", "attn_fwd_fp8qk"])
def test_int8_argument_errors(L, name):
    fn = getattr(L, name)
    need = L.attn_int8qk_workspace_bytes(1, 1, 64, 64)
    args = [FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, 1, 1, 64, 64, 0.125]
    assert fn(*args, None, need, None) == EWS
    assert fn(*args, FAKE + 0x8000, need - 1, None) == EWS
    assert fn(*args, FAKE + 0x8010, need, None) == EWS   # not 256-aligned
    bad = list(args); bad[7] = 80
    assert fn(*bad, FAKE + 0x8000, need, None) == EUNSUP
    bad = list(args); bad[0] = None
    assert fn(*bad, FAKE + 0x8000, need, None) == EINVAL


def _contig(H, S, D):
    return [H * S * D, S * D, D] * 4


def _ex(L, strides=None, out_dtype=0, lse=None, q=FAKE, o=FAKE + 0x3000, B=1, H=2, S=64, D=64,
        int8=False, fp8=False):
    st = _contig(H, S, D) if strides is None else strides
    arr = (ctypes.c_int64 * 12)(*st) if st is not False else None
    args = [q, FAKE + 0x1000, FAKE + 0x2000, o, out_dtype, lse, arr, B, H, S, D, 0.125]
    if int8:
        need = L.attn_int8qk_workspace_bytes(B, H, S, D)
        fn = L.attn_fwd_fp8qk_ex if fp8 else L.attn_fwd_int8qk_ex
        return fn(*args, FAKE + 0x8000, need - 1, None)
    return L.attn_fwd_bf16_ex(*args, None)


@pytest.mark.parametrize("int8,fp8", [(False, False), (True, False), (True, True)])
def test_ex_argument_errors(L, int8, fp8):
    # every bad call fails validation before anything is launched; the int8 calls get a too
    # small workspace, so a call that passed validation would return EWORKSPACE, not launch
    ok = EWS if int8 else None
    assert _ex(L, strides=False, int8=int8, fp8=fp8) == EINVAL                     # NULL strides
    for bad in (-1, 2, 7):
        assert _ex(L, out_dtype=bad, int8=int8, fp8=fp8) == EINVAL
    assert _ex(L, q=None, int8=int8, fp8=fp8) == EINVAL
    assert _ex(L, o=FAKE, int8=int8, fp8=fp8) == EINVAL                           # o aliases q
    assert _ex(L, q=FAKE + 8, int8=int8, fp8=fp8) == EINVAL                       # misaligned
    assert _ex(L, lse=FAKE + 0x3000, int8=int8, fp8=fp8) == EINVAL                # lse aliases o
    assert _ex(L, lse=FAKE + 0x4002, int8=int8, fp8=fp8) == EINVAL                # lse misaligned
    assert _ex(L, D=96, strides=_contig(2, 64, 96), int8=int8, fp8=fp8) == EUNSUP
    for t in range(4):
        for a in range(3):
            st = _contig(2, 64, 64); st[3 * t + a] = -64
            assert _ex(L, strides=st, int8=int8, fp8=fp8) == EINVAL               # negative stride
            st = _contig(2, 64, 64); st[3 * t + a] += 2
            assert _ex(L, strides=st, int8=int8, fp8=fp8) == EINVAL               # not 16-byte steps
    for t in range(3):
        st = _contig(2, 64, 64); st[3 * t + 2] = 1 << 24
        assert _ex(L, strides=st, int8=int8, fp8=fp8) == EINVAL                   # token stride too big
    # fp32 output: strides in steps of 4 elements pass validation; bf16 output needs 8
    st = _contig(2, 64, 64); st[11] = 68
    if int8:
        assert _ex(L, strides=st, int8=True, fp8=fp8) == ok
        assert _ex(L, strides=st, out_dtype=1, int8=True, fp8=fp8) == EINVAL
        # the output's token stride has no 2^24 limit; stride 0 (broadcast inputs) is valid
        st = _contig(2, 64, 64); st[11] = 1 << 30; st[0] = st[1] = 0
        assert _ex(L, strides=st, int8=True, fp8=fp8) == ok
        assert _ex(L, lse=FAKE + 0x4004, int8=True, fp8=fp8) == ok
    else:
        assert _ex(L, strides=st, out_dtype=1) == EINVAL


def test_rel_l1_argument_errors(L):
    need = L.resid_rel_l1_workspace_bytes(100)
    assert L.resid_rel_l1(None, FAKE, 100, FAKE + 0x1000, FAKE + 0x2000, need, None) == EINVAL
    assert L.resid_rel_l1(FAKE, FAKE + 0x100, 0, FAKE + 0x1000, FAKE + 0x2000, need, None) == EINVAL
    assert L.resid_rel_l1(FAKE + 2, FAKE + 0x100, 100, FAKE + 0x1000, FAKE + 0x2000, need, None) == EINVAL
    assert L.resid_rel_l1(FAKE, FAKE + 0x100, 100, FAKE + 0x1000, None, need, None) == EWS
    assert L.resid_rel_l1(FAKE, FAKE + 0x100, 100, FAKE + 0x1000, FAKE + 0x2000, need - 1, None) == EWS


def test_rel_l1_noalloc_argument_errors(L):
    # rejected before any HIP call (the device array is only looked up for a valid call)
    assert L.resid_rel_l1_noalloc(None, FAKE, 100, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, None, 100, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, FAKE + 0x100, 100, None, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, FAKE + 0x100, 0, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, FAKE + 0x100, -5, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE + 2, FAKE + 0x100, 100, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, FAKE + 0x108, 100, FAKE + 0x1000, None) == EINVAL
    assert L.resid_rel_l1_noalloc(FAKE, FAKE + 0x100, 100, FAKE + 0x1002, None) == EINVAL


def test_mfma_probe_argument_errors(L):
    assert L.ditattn_mfma_probe(2, 1, 10, FAKE, None) == EINVAL
    assert L.ditattn_mfma_probe(-1, 1, 10, FAKE, None) == EINVAL
    assert L.ditattn_mfma_probe(0, 2, 10, FAKE, None) == EINVAL
    assert L.ditattn_mfma_probe(0, 1, 0, FAKE, None) == EINVAL
    assert L.ditattn_mfma_probe(1, 0, 10, None, None) == EINVAL
    assert L.ditattn_mfma_probe(1, 0, 10, FAKE + 4, None) == EINVAL


def test_quant_probe_workspace_and_errors(L):
    assert L.attn_quant_probe_splits(1, 24, 118800, 128, 256) == 10   # 24 workgroups per chunk
    assert L.attn_quant_probe_splits(1, 2, 1000, 64, 100) == 1        # chunks >= ~1024 keys
    assert L.attn_quant_probe_splits(1, 1, 1 << 20, 64, 64) == 16     # at most 16
    assert L.attn_quant_probe_splits(1, 1, 100, 64, 101) == 0
    assert L.attn_quant_probe_workspace_bytes(1, 24, 4608, 128, 0) == 0
    assert L.attn_quant_probe_workspace_bytes(1, 24, 4608, 128, 4609) == 0
    assert L.attn_quant_probe_workspace_bytes(1, 24, 4608, 96, 64) == 0
    need = L.attn_quant_probe_workspace_bytes(1, 2, 4096, 64, 64)
    # at least the chunk outputs of one split and the per-head sums
    assert need >= 1 * 2 * 64 * 64 * 4 + 2 * 16 and need % 256 == 0
    st = (ctypes.c_int64 * 12)(*_contig(2, 4096, 64))
    Q, K, V, O, E, W = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000, FAKE + 0x4000, FAKE + 0x8000

    def call(n_rows=64, err=E, ws=W, ws_bytes=need, o=O, dtype=0, strides=st, D=64):
        return L.attn_quant_probe(Q, K, V, o, dtype, strides, 1, 2, 4096, D, 0.125, n_rows, err,
                                  ws, ws_bytes, None)
    assert call(n_rows=0) == EINVAL
    assert call(n_rows=4097) == EINVAL
    assert call(err=None) == EINVAL
    assert call(err=E + 2) == EINVAL
    assert call(o=Q) == EINVAL
    assert call(dtype=3) == EINVAL
    assert call(strides=None) == EINVAL
    assert call(D=80) == EUNSUP
    assert call(ws=None) == EWS
    assert call(ws_bytes=need - 1) == EWS
    assert call(ws=W + 16) == EWS


def test_fbcache_struct_layout_matches_header():
    import diffusion_transformer_attention_amd as dta
    assert ctypes.sizeof(dta.FBCacheConfig) == 16
    cfg = dta.FBCacheConfig()
    assert (round(cfg.residual_diff_threshold, 6), cfg.max_warmup_steps, cfg.max_cached_steps,
            cfg.max_continuous_cached_steps) == (0.24, 4, -1, 3)
    text = open(HEADER).read()
    body = text[text.index("typedef struct ditattn_fbcache_state"):]
    body = body[:body.index("} ditattn_fbcache_state;")]
    # 4 int32 + 1 float + 3 reserved int32 = 32 bytes, the size fbcache_state() allocates
    assert body.count("int32_t") == 5 and "reserved[3]" in body and body.count("float") == 1


def test_fbcache_argument_errors(L):
    import diffusion_transformer_attention_amd as dta
    need = L.resid_rel_l1_workspace_bytes(100)
    R, P, ST, WS = FAKE, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000

    def call(cfg=None, resid=R, prev=P, n=100, state=ST, ws=WS, ws_bytes=need):
        c = dta.FBCacheConfig() if cfg is None else cfg
        return L.fbcache_decide(resid, prev, n, ctypes.byref(c), state, ws, ws_bytes, None)

    assert L.fbcache_decide(R, P, 100, None, ST, WS, need, None) == EINVAL   # no config
    assert call(resid=None) == EINVAL
    assert call(state=None) == EINVAL
    assert call(n=0) == EINVAL
    assert call(resid=R + 8) == EINVAL
    assert call(prev=P + 8) == EINVAL
    assert call(state=ST + 2) == EINVAL
    for bad in (dta.FBCacheConfig(residual_diff_threshold=-0.1),
                dta.FBCacheConfig(residual_diff_threshold=float("nan")),
                dta.FBCacheConfig(residual_diff_threshold=float("inf")),
                dta.FBCacheConfig(max_warmup_steps=-1),
                dta.FBCacheConfig(max_cached_steps=-2),
                dta.FBCacheConfig(max_continuous_cached_steps=-2)):
        assert call(cfg=bad) == EINVAL
    assert call(ws=None) == EWS
    assert call(ws_bytes=need - 1) == EWS


def test_resid_addsub_argument_errors(L):
    A, B, O = FAKE, FAKE + 0x1000, FAKE + 0x2000
    for fn in (L.resid_add, L.resid_sub):
        assert fn(None, B, O, 64, None) == EINVAL
        assert fn(A, B, None, 64, None) == EINVAL
        assert fn(A, B, O, 0, None) == EINVAL
        assert fn(A + 2, B, O, 64, None) == EINVAL
        assert fn(A, B, O + 8, 64, None) == EINVAL
        assert fn(A, B, A + 16, 64, None) == EINVAL      # out overlaps a partly
        assert fn(A, B, B - 16, 64, None) == EINVAL      # out overlaps b partly


def test_binding_rejects_cpu_tensors():
    import torch
    import diffusion_transformer_attention_amd as dta
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dta.attn_fwd_bf16(x, x, x)
    with pytest.raises(ValueError):
        dta.attn_fwd_bf16(x, x, x, out_dtype=torch.bfloat16, lse=True)
    with pytest.raises(ValueError):
        dta.attn_fwd_int8qk(x, x, x, lse=True)
    with pytest.raises(ValueError):
        dta.resid_rel_l1(x, x)
    with pytest.raises(ValueError):
        dta.resid_add(x, x)
    with pytest.raises(ValueError):
        dta.fbcache_decide(x, None, torch.zeros(8, dtype=torch.int32))


def test_binding_strides_of_views():
    """The (batch, head, token) strides the binding hands to the extended calls."""
    import torch
    import diffusion_transformer_attention_amd as dta
    B, S, H, D = 2, 40, 3, 64
    bshd = torch.zeros(B, S, H, D, dtype=torch.bfloat16).transpose(1, 2)
    assert dta._bhs_strides(bshd) == [S * H * D, D, H * D]
    qkv = torch.zeros(B, S, 3, H, D, dtype=torch.bfloat16)        # fused QKV projection
    assert dta._bhs_strides(qkv[:, :, 1].transpose(1, 2)) == [S * 3 * H * D, D, 3 * H * D]
    one = torch.zeros(1, 1, S, D, dtype=torch.bfloat16)
    assert dta._bhs_strides(one) == [0, 0, D]                     # size-1 axes never stepped
