"""Python binding of libditattn.so, the MI355X (gfx950) DiT attention library.

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
PyTorch provides device memory and the current stream; tensors are checked for device,
dtype, contiguity and shape here, the library validates the rest and returns a status that
is raised as DitAttnError.  There is no fallback: if the library is not built, loading it
raises.

Entry points (same names as the C ABI in include/ditattn.h):

  attn_fwd_bf16(q, k, v, out=None, scale=None, workspace=None) -> out
  attn_fwd_int8qk(q, k, v, out=None, scale=None, workspace=None) -> out
  attn_fwd_fp8qk(q, k, v, out=None, scale=None, workspace=None) -> out
  attn_fwd_fp8(q, k, v, out=None, scale=None, workspace=None) -> out   (fp8 QK and PV, D = 128)
  resid_rel_l1(a, b, out=None, workspace=None) -> out (fp32 device scalar, shape [1])
  resid_rel_l1_noalloc(a, b, out) -> out (same result; no workspace, no allocation)
  attn_quant_probe(q, k, v, o_q, n_rows=256, scale=None) -> err (fp32 [1 + B*H])
  fbcache_decide(resid, prev_resid, state, config, workspace=None) -> state
  resid_add(a, b, out=None) -> out;  resid_sub(a, b, out=None) -> out
  mfma_probe(dtype, random_operands, iters) -> clocks   (calibration, not the attention path)

plus helpers for the workspaces (bf16_workspace, int8qk_workspace, int8qk_views), the First
Block Cache state (FBCacheConfig, fbcache_state, fbcache_state_values) and the library path.

The attention calls also take strided [B, H, S, D] views (channel axis contiguous), for
instance q.transpose(1, 2) of a [B, S, H, D] tensor or a slice of a fused QKV projection, an
output dtype (out_dtype=torch.bfloat16, or a bf16 `out`) and `lse` (a fp32 [B, H, S] tensor,
or lse=True to allocate one), which return (out, lse); those go through the C ABI's
attn_fwd_bf16_ex / attn_fwd_int8qk_ex, the plain contiguous fp32 case through the plain calls.
With a workspace (the default) the bf16 call goes through attn_fwd_bf16_ws, which shares the
last, partly filled round of query tiles out over every CU.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loaded first: the library then binds to the HIP runtime torch already holds

__all__ = ["attn_fwd_bf16", "bf16_workspace", "bf16_workspace_bytes", "attn_fwd_int8qk", "attn_fwd_fp8qk", "attn_fwd_fp8", "fp8_workspace",
           "fp8_views", "resid_rel_l1", "resid_rel_l1_noalloc", "int8qk_workspace",
           "int8qk_views", "int8qk_workspace_bytes", "rel_l1_workspace_bytes", "fbcache_decide",
           "resid_add", "resid_sub", "FBCacheConfig", "fbcache_state", "fbcache_state_values",
           "attn_quant_probe", "quant_probe_workspace_bytes", "quant_probe_views",
           "mfma_probe", "mfma_probe_flops", "lib", "LIB_PATH", "DitAttnError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")

STATUS = {0: "DITATTN_OK", -1: "DITATTN_EINVAL", -2: "DITATTN_EUNSUPPORTED",
          -3: "DITATTN_EWORKSPACE", -4: "DITATTN_EHIP"}

_lib = None


class FBCacheConfig(ctypes.Structure):
    """ditattn_fbcache_config: the cache policy (defaults: the DBCache defaults)."""
    _fields_ = [("residual_diff_threshold", ctypes.c_float), ("max_warmup_steps", ctypes.c_int32),
                ("max_cached_steps", ctypes.c_int32), ("max_continuous_cached_steps", ctypes.c_int32)]

    def __init__(self, residual_diff_threshold=0.24, max_warmup_steps=4, max_cached_steps=-1,
                 max_continuous_cached_steps=3):
        super().__init__(residual_diff_threshold, max_warmup_steps, max_cached_steps,
                         max_continuous_cached_steps)


class DitAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libditattn.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m diffusion_transformer_attention_amd.build`")
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C ABI's signatures (include/ditattn.h) on a loaded copy of the library."""
    vp, i, f, sz, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_int64
    L.attn_fwd_bf16.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp]
    L.attn_fwd_bf16.restype = i
    L.attn_int8qk_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_int8qk_workspace_bytes.restype = sz
    L.attn_int8qk_workspace_offsets.argtypes = [i, i, i, i, ctypes.POINTER(sz)]
    L.attn_int8qk_workspace_offsets.restype = sz
    L.attn_fwd_int8qk.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_int8qk.restype = i
    p64 = ctypes.POINTER(i64)
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_fwd_fp8_ex.argtypes = [vp, vp, vp, vp, i, vp, p64, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_fp8_ex.restype = i
    L.attn_fp8_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_fp8_workspace_bytes.restype = sz
    L.attn_fp8_workspace_offsets.argtypes = [i, i, i, i, ctypes.POINTER(sz)]
    L.attn_fp8_workspace_offsets.restype = sz
    L.attn_fwd_fp8qk.argtypes = [vp, vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_fp8qk.restype = i
    L.attn_fwd_fp8qk_ex.argtypes = [vp, vp, vp, vp, i, vp, p64, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_fp8qk_ex.restype = i
    L.attn_fwd_bf16_ex.argtypes = [vp, vp, vp, vp, i, vp, p64, i, i, i, i, f, vp]
    L.attn_fwd_bf16_ex.restype = i
    L.attn_bf16_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_bf16_workspace_bytes.restype = sz
    L.attn_fwd_bf16_ws.argtypes = [vp, vp, vp, vp, i, vp, p64, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_bf16_ws.restype = i
    L.attn_fwd_int8qk_ex.argtypes = [vp, vp, vp, vp, i, vp, p64, i, i, i, i, f, vp, sz, vp]
    L.attn_fwd_int8qk_ex.restype = i
    L.resid_rel_l1_workspace_bytes.argtypes = [i64]
    L.resid_rel_l1_workspace_bytes.restype = sz
    L.resid_rel_l1.argtypes = [vp, vp, i64, vp, vp, sz, vp]
    L.resid_rel_l1.restype = i
    L.resid_rel_l1_noalloc.argtypes = [vp, vp, i64, vp, vp]
    L.resid_rel_l1_noalloc.restype = i
    L.attn_quant_probe_splits.argtypes = [i, i, i, i, i]
    L.attn_quant_probe_splits.restype = i
    L.attn_quant_probe_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_quant_probe_workspace_bytes.restype = sz
    L.attn_quant_probe.argtypes = [vp, vp, vp, vp, i, p64, i, i, i, i, f, i, vp, vp, sz, vp]
    L.attn_quant_probe.restype = i
    L.fbcache_decide.argtypes = [vp, vp, i64, ctypes.POINTER(FBCacheConfig), vp, vp, sz, vp]
    L.fbcache_decide.restype = i
    L.resid_add.argtypes = [vp, vp, vp, i64, vp]
    L.resid_add.restype = i
    L.resid_sub.argtypes = [vp, vp, vp, i64, vp]
    L.resid_sub.restype = i
    L.ditattn_mfma_probe.argtypes = [i, i, i, vp, vp]
    L.ditattn_mfma_probe.restype = i
    L.ditattn_status_string.argtypes = [i]
    L.ditattn_status_string.restype = ctypes.c_char_p
    return L


def _check(status: int):
    if status != 0:
        raise DitAttnError(status, lib().ditattn_status_string(status).decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


OUT_F32, OUT_BF16 = 0, 1


def _qkv_shape(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{name} must be a 4-D bf16 CUDA tensor [B, H, S, D] "
                             "with a contiguous channel axis")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must have the same shape [B, H, S, D]")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on the same device")
    return tuple(int(x) for x in q.shape)


def _bhs_strides(t):
    """(batch, head, token) element strides; a size-1 axis is never stepped, so it gets 0."""
    return [0 if t.shape[d] == 1 else int(t.stride(d)) for d in range(3)]


def _attn_args(q, k, v, out, out_dtype, lse):
    """Shape, output tensor, lse tensor (or None) and whether the extended call is needed."""
    B, H, S, D = _qkv_shape(q, k, v)
    if out is not None:
        if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (B, H, S, D) \
                or out.stride(3) != 1 or out.device != q.device:
            raise ValueError(f"out must be a fp32 or bf16 tensor of shape {(B, H, S, D)} on "
                             "q's device with a contiguous channel axis")
        if out_dtype is not None and out.dtype != out_dtype:
            raise ValueError("out_dtype differs from out.dtype")
    else:
        dt = torch.float32 if out_dtype is None else out_dtype
        if dt not in (torch.float32, torch.bfloat16):
            raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
        if q.stride(1) < q.stride(2):   # heads interleaved per token: keep q's [B, S, H, D] order
            out = torch.empty((B, S, H, D), dtype=dt, device=q.device).transpose(1, 2)
        else:
            out = torch.empty((B, H, S, D), dtype=dt, device=q.device)
    if lse is True:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S)
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError(f"lse must be a contiguous fp32 tensor of shape {(B, H, S)}")
    plain = (lse is None and out.dtype == torch.float32
             and all(t.is_contiguous() for t in (q, k, v, out)))
    return (B, H, S, D), out, lse, plain


def _strides_arg(q, k, v, out):
    return (ctypes.c_int64 * 12)(*(_bhs_strides(q) + _bhs_strides(k) + _bhs_strides(v)
                                   + _bhs_strides(out)))


def bf16_workspace_bytes(B, H, S, D) -> int:
    return int(lib().attn_bf16_workspace_bytes(B, H, S, D))


def bf16_workspace(B, H, S, D, device) -> torch.Tensor:
    """A uint8 device buffer large enough for attn_fwd_bf16's split of the last round."""
    n = bf16_workspace_bytes(B, H, S, D)
    if n == 0:
        raise DitAttnError(-1, "invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def attn_fwd_bf16(q, k, v, out=None, scale=None, *, out_dtype=None, lse=None, workspace=None):
    """Exact attention O = softmax(Q K^T * scale) V on bf16 [B,H,S,D] views.

    workspace: a bf16_workspace buffer, None to allocate one, or False for the calls that take
    none (whole tiles only: the last round of query tiles may leave CUs idle).
    Returns out (fp32 unless out_dtype / out say bf16), or (out, lse) when lse is given."""
    (B, H, S, D), out, lse_t, plain = _attn_args(q, k, v, out, out_dtype, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is not False:
        if workspace is None:
            workspace = bf16_workspace(B, H, S, D, q.device)
        if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
        _check(lib().attn_fwd_bf16_ws(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out),
            OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32, _ptr(lse_t),
            _strides_arg(q, k, v, out), B, H, S, D, scale, _ptr(workspace), workspace.numel(),
            _stream(q)))
    elif plain:
        _check(lib().attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, S, D, scale,
                                   _stream(q)))
    else:
        _check(lib().attn_fwd_bf16_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out),
            OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32, _ptr(lse_t),
            _strides_arg(q, k, v, out), B, H, S, D, scale, _stream(q)))
    return out if lse_t is None else (out, lse_t)


def int8qk_workspace_bytes(B, H, S, D) -> int:
    return int(lib().attn_int8qk_workspace_bytes(B, H, S, D))


def int8qk_workspace(B, H, S, D, device) -> torch.Tensor:
    """A uint8 device buffer large enough for attn_fwd_int8qk on this shape."""
    n = int8qk_workspace_bytes(B, H, S, D)
    if n == 0:
        raise DitAttnError(-1, "invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def int8qk_views(workspace: torch.Tensor, B, H, S, D) -> dict:
    """Views of the workspace segments: k_mean, q_scale, k_scale, q_codes, k_codes."""
    off = (ctypes.c_size_t * 6)()
    total = lib().attn_int8qk_workspace_offsets(B, H, S, D, off)
    if total == 0 or workspace.numel() < total:
        raise DitAttnError(-3, "workspace too small for this shape")
    nqb, nkb = -(-S // 128), -(-S // 64)

    def seg(i, dtype, shape):
        n = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
        return workspace[off[i]:off[i] + n].view(dtype).view(shape)

    return {"k_mean": seg(0, torch.float32, (B, H, D)),
            "q_scale": seg(1, torch.float32, (B, H, nqb)),
            "k_scale": seg(2, torch.float32, (B, H, nkb)),
            "q_codes": seg(3, torch.int8, (B, H, S, D)),
            "k_codes": seg(4, torch.int8, (B, H, S, D))}


def _attn_q8(plain_fn, ex_fn, q, k, v, out, scale, workspace, out_dtype, lse, ws_fn=None):
    (B, H, S, D), out, lse_t, plain = _attn_args(q, k, v, out, out_dtype, lse)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if workspace is None:
        workspace = (ws_fn or int8qk_workspace)(B, H, S, D, q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 CUDA tensor")
    if plain:
        _check(plain_fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, S, D, scale,
                        _ptr(workspace), workspace.numel(), _stream(q)))
    else:
        _check(ex_fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out),
                     OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32, _ptr(lse_t),
                     _strides_arg(q, k, v, out), B, H, S, D, scale, _ptr(workspace),
                     workspace.numel(), _stream(q)))
    return out if lse_t is None else (out, lse_t)


def attn_fwd_int8qk(q, k, v, out=None, scale=None, workspace=None, *, out_dtype=None, lse=None):
    """int8-QK attention (K smoothed by its channel mean, per-block int8 Q/K, bf16 PV).

    Arguments and result as attn_fwd_bf16; lse is that of the quantized scores."""
    return _attn_q8(lib().attn_fwd_int8qk, lib().attn_fwd_int8qk_ex, q, k, v, out, scale,
                    workspace, out_dtype, lse)


def attn_fwd_fp8qk(q, k, v, out=None, scale=None, workspace=None, *, out_dtype=None, lse=None):
    """fp8-QK attention: as attn_fwd_int8qk with e4m3 codes (scale = amax / 448) and QK on the
    fp8 matrix cores.  The workspace is the int8 call's (int8qk_workspace); its code views hold
    e4m3 bytes."""
    return _attn_q8(lib().attn_fwd_fp8qk, lib().attn_fwd_fp8qk_ex, q, k, v, out, scale,
                    workspace, out_dtype, lse)


def fp8_workspace(B, H, S, D, device) -> torch.Tensor:
    """A uint8 device buffer large enough for attn_fwd_fp8 on this shape."""
    n = int(lib().attn_fp8_workspace_bytes(B, H, S, D))
    if n == 0:
        raise DitAttnError(-1, "invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def fp8_views(workspace: torch.Tensor, B, H, S, D) -> dict:
    """Views of the attn_fwd_fp8 workspace: as int8qk_views (codes as uint8 e4m3 bytes) plus
    v_scale [B, H, D] and v_codes [B, H, S, D]."""
    off = (ctypes.c_size_t * 9)()
    total = lib().attn_fp8_workspace_offsets(B, H, S, D, off)
    if total == 0 or workspace.numel() < total:
        raise DitAttnError(-3, "workspace too small for this shape")
    views = int8qk_views(workspace, B, H, S, D)
    views["q_codes"] = views["q_codes"].view(torch.uint8)
    views["k_codes"] = views["k_codes"].view(torch.uint8)
    views["v_scale"] = workspace[off[6]:off[6] + B * H * D * 4].view(torch.float32).view(B, H, D)
    views["v_codes"] = workspace[off[7]:off[7] + B * H * S * D].view(B, H, S, D)
    return views


def attn_fwd_fp8(q, k, v, out=None, scale=None, workspace=None, *, out_dtype=None, lse=None):
    """Attention with fp8 e4m3 codes for Q, K (per block) and V (per channel): both products on
    the fp8 matrix cores (D = 128).  Arguments and result as attn_fwd_bf16; the workspace comes
    from fp8_workspace."""
    return _attn_q8(lib().attn_fwd_fp8, lib().attn_fwd_fp8_ex, q, k, v, out, scale, workspace,
                    out_dtype, lse, ws_fn=fp8_workspace)


def rel_l1_workspace_bytes(n: int) -> int:
    return int(lib().resid_rel_l1_workspace_bytes(n))


def resid_rel_l1(a, b, out=None, workspace=None):
    """sum|a - b| / sum|b| over two equally shaped bf16 CUDA tensors -> fp32 device tensor [1]."""
    for name, t in (("a", a), ("b", b)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    n = a.numel()
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=a.device)
    if workspace is None:
        workspace = torch.empty(max(rel_l1_workspace_bytes(n), 1), dtype=torch.uint8, device=a.device)
    _check(lib().resid_rel_l1(_ptr(a), _ptr(b), n, _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream(a)))
    return out


def resid_rel_l1_noalloc(a, b, out):
    """resid_rel_l1 through the allocation-free entry point: the caller passes the fp32 device
    tensor [1] for the result; the library keeps the partial sums in its own static device
    array (calls that overlap on one GPU race)."""
    for name, t in (("a", a), ("b", b)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    if not out.is_cuda or out.dtype != torch.float32 or out.numel() < 1:
        raise ValueError("out must be an fp32 CUDA tensor of at least one element")
    _check(lib().resid_rel_l1_noalloc(_ptr(a), _ptr(b), a.numel(), _ptr(out), _stream(a)))
    return out


# ---- quantization-error probe ---------------------------------------------------------------

def quant_probe_workspace_bytes(B, H, S, D, n_rows) -> int:
    return int(lib().attn_quant_probe_workspace_bytes(B, H, S, D, n_rows))


def quant_probe_views(workspace, B, H, S, D, n_rows) -> dict:
    """Views of the probe workspace: the chunk outputs `part` [B, ns + 1, H, n_rows, D], their
    log-sum-exps `lse` [B, ns + 1, H, n_rows] and the key range [start, stop) of each chunk
    that holds keys (`chunks`; the last slot is used only when ns L < S)."""
    ns = int(lib().attn_quant_probe_splits(B, H, S, D, n_rows))
    if ns == 0:
        raise DitAttnError(-1, "invalid shape or n_rows")
    L = (S // ns) // 64 * 64
    if ns == 1 or L == 0:
        L = S
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    n_part = B * (ns + 1) * H * n_rows * D
    part = workspace[:n_part * 4].view(torch.float32).view(B, ns + 1, H, n_rows, D)
    off = al(n_part * 4)
    lse = workspace[off:off + B * (ns + 1) * H * n_rows * 4].view(torch.float32)
    lse = lse.view(B, ns + 1, H, n_rows)
    chunks = [(c * L, (c + 1) * L) for c in range(ns)]
    if ns * L < S:
        chunks.append((ns * L, S))
    return {"part": part, "lse": lse, "chunks": chunks}


def attn_quant_probe(q, k, v, o_q, n_rows=256, scale=None, err=None, workspace=None):
    """Relative L2 error of a quantized call's output o_q (fp32 or bf16 [B,H,S,D] view) against
    the bf16 path on n_rows evenly spaced query rows per (b, h).  Returns err (fp32 device
    tensor [1 + B*H]): err[0] over all rows, err[1 + b*H + h] per head."""
    B, H, S, D = _qkv_shape(q, k, v)
    if o_q.dtype not in (torch.float32, torch.bfloat16) or tuple(o_q.shape) != (B, H, S, D) \
            or o_q.stride(3) != 1 or o_q.device != q.device:
        raise ValueError(f"o_q must be a fp32 or bf16 tensor of shape {(B, H, S, D)} on q's device")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if err is None:
        err = torch.empty(1 + B * H, dtype=torch.float32, device=q.device)
    if workspace is None:
        n = quant_probe_workspace_bytes(B, H, S, D, n_rows)
        if n == 0:
            raise DitAttnError(-1, "invalid shape or n_rows")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(lib().attn_quant_probe(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o_q), OUT_BF16 if o_q.dtype == torch.bfloat16 else OUT_F32,
        _strides_arg(q, k, v, o_q), B, H, S, D, scale, n_rows, _ptr(err), _ptr(workspace),
        workspace.numel(), _stream(q)))
    return err


# ---- First Block Cache ----------------------------------------------------------------------

def fbcache_state(device) -> torch.Tensor:
    """A zeroed ditattn_fbcache_state (32 bytes of device memory) for a new run."""
    return torch.zeros(8, dtype=torch.int32, device=device)


def fbcache_state_values(state: torch.Tensor) -> dict:
    """The state's fields, read back to the host (synchronises with the state's stream)."""
    h = state.cpu()
    return {"steps": int(h[0]), "cached_steps": int(h[1]), "continuous_cached_steps": int(h[2]),
            "use_cache": int(h[3]), "diff": float(h[4:5].view(torch.float32)[0])}


def _bf16_flat(name, t):
    if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")


def fbcache_decide(resid, prev_resid, state, config=None, workspace=None):
    """One step's cache decision on `state` (from fbcache_state); prev_resid None = no reference.
    The decision stays on the device: state[3] (1 = reuse the cache)."""
    _bf16_flat("resid", resid)
    if prev_resid is not None:
        _bf16_flat("prev_resid", prev_resid)
        if prev_resid.shape != resid.shape:
            raise ValueError("resid and prev_resid must have the same shape")
    if state.dtype != torch.int32 or state.numel() != 8 or not state.is_cuda or not state.is_contiguous():
        raise ValueError("state must come from fbcache_state()")
    cfg = FBCacheConfig() if config is None else config
    n = resid.numel()
    if prev_resid is not None and workspace is None:
        workspace = torch.empty(max(rel_l1_workspace_bytes(n), 1), dtype=torch.uint8, device=resid.device)
    ws_n = workspace.numel() if workspace is not None else 0
    _check(lib().fbcache_decide(_ptr(resid), _ptr(prev_resid), n, ctypes.byref(cfg), _ptr(state),
                                _ptr(workspace), ws_n, _stream(resid)))
    return state


def _resid_op(fn, a, b, out):
    _bf16_flat("a", a)
    _bf16_flat("b", b)
    if a.shape != b.shape:
        raise ValueError("a and b must have the same shape")
    if out is None:
        out = torch.empty_like(a)
    else:
        _bf16_flat("out", out)
        if out.shape != a.shape:
            raise ValueError("out must have the shape of a")
    _check(fn(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(a)))
    return out


def resid_add(a, b, out=None):
    """out = a + b over bf16 tensors, each value rounded once (out may be a or b)."""
    return _resid_op(lib().resid_add, a, b, out)


def resid_sub(a, b, out=None):
    """out = a - b over bf16 tensors, each value rounded once (out may be a or b)."""
    return _resid_op(lib().resid_sub, a, b, out)


# ---- calibration (not part of the attention path) ------------------------------------------

MFMA_PROBE_WORKGROUPS = 1024


def mfma_probe_flops(dtype: str, iters: int) -> float:
    """Work of one ditattn_mfma_probe launch: flops (bf16) or integer ops (int8)."""
    per = 32 * 32 * (16 if dtype == "bf16" else 32) * 2
    return float(MFMA_PROBE_WORKGROUPS) * 8 * iters * 8 * per


def mfma_probe(dtype: str = "bf16", random_operands: bool = True, iters: int = 1000, clocks=None):
    """Launch the matrix-core calibration kernel on the current stream; returns the int64
    clocks tensor [1024, 2] (shader clocks, 100 MHz reference clocks per workgroup)."""
    if dtype not in ("bf16", "int8"):
        raise ValueError("dtype must be 'bf16' or 'int8'")
    if clocks is None:
        clocks = torch.empty((MFMA_PROBE_WORKGROUPS, 2), dtype=torch.int64, device="cuda")
    _check(lib().ditattn_mfma_probe(0 if dtype == "bf16" else 1, 1 if random_operands else 0,
                                    int(iters), _ptr(clocks), _stream(clocks)))
    return clocks
