"""int8-QK attention: K smoothing, per-block symmetric int8 quantization, quantized attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages motivate the method and fix two of its rules:

* 8-bit quantized attention (SageAttention) as a DiT attention backend, with head-level
  parallelism leaving each device the full sequence -- "TMAP platform image-to-video
  inference acceleration" page, section on combining with the SageAttention operator; its
  results section reports attention time cut to one third; the "Diffusion Attention Backends"
  page lists SAGE_ATTN and warns that its quality must be validated per model.
* A quantization scale computed from an all-zero group of values is zero, the division by it
  gives NaN and the output turns black -- same TMAP page, section on operator details; the fix
  is in the scale logic.  Here: a group whose absolute maximum is 0 gets scale 1.0 (any
  positive value yields the same all-zero codes, hence the same output).

The rest is this library's stated contract (the pages leave it open):

1. K channel mean over the sequence, per (b, h, d): the exact sum of the bf16 values
   (math.fsum, correctly rounded to fp64), divided by S in fp64, rounded once to fp32.
2. Smoothed keys Ks = fp32(K) - mean, one fp32 subtraction.  Subtracting the same vector from
   every key shifts all scores of a query row by one constant, which the softmax cancels, so
   the attention output is unchanged; it only shrinks the range the int8 grid must cover.
   Q is not smoothed and the softmax scale is not folded into the codes.
3. Blocks: Q in blocks of 128 consecutive tokens, K in blocks of 64, each within one (b, h);
   a tail block holds only the valid tokens.
4. Per block: amax = max |x| over the block's tokens and all D channels;
   scale = amax / 127 as one IEEE fp32 division; amax == 0 gives scale = 1.0.
5. code = clamp(round_half_even(x / scale), -127, 127), x / scale one IEEE fp32 division.
6. Attention on the codes: s_ij = (sum_d qc_id * kc_jd) * sq[i // 128] * sk[j // 64] * scale,
   the integer dot product exact; softmax and the product with V (bf16 values) as in exact
   attention, all in fp64.

The fp8 variant (end of the module) keeps rules 1-3 and 6 and replaces 4-5 by e4m3 codes:
scale = amax / 448 and one rounding of x / scale to the nearest e4m3 value.
"""
from __future__ import annotations

import math

import numpy as np

QMAX = 127
Q_BLOCK = 128
K_BLOCK = 64


def k_channel_mean(k) -> np.ndarray:
    """Per-(b, h, d) mean of K over the token axis -> float32 [B, H, D] (rule 1).

    k: [B, H, S, D] fp64 holding bf16 values exactly.
    """
    k = np.asarray(k, dtype=np.float64)
    B, H, S, D = k.shape
    out = np.empty((B, H, D), dtype=np.float32)
    for b in range(B):
        for h in range(H):
            cols = np.ascontiguousarray(k[b, h].T)
            for d in range(D):
                out[b, h, d] = np.float32(math.fsum(cols[d].tolist()) / S)
    return out


def smooth_k(k, kmean) -> np.ndarray:
    """Ks = fp32(K) - mean, in fp32 (rule 2).  k: [B, H, S, D]; kmean: float32 [B, H, D]."""
    kf = np.asarray(k, dtype=np.float64).astype(np.float32)
    return kf - np.asarray(kmean, dtype=np.float32)[:, :, None, :]


def _block_scale(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    scale = amax / np.float32(QMAX)
    return np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)


def quantize_blocks(x, block: int):
    """Symmetric int8 codes and per-block scales (rules 3-5).

    x: float32 [B, H, S, D].  Returns (codes int8 [B, H, S, D], scales float32 [B, H, nblk])
    with nblk = ceil(S / block).
    """
    x = np.asarray(x, dtype=np.float32)
    B, H, S, D = x.shape
    nblk = -(-S // block)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    codes = np.empty((B, H, S, D), dtype=np.int8)
    for t in range(nblk):
        blk = x[:, :, t * block:min(S, (t + 1) * block)]
        scale = _block_scale(np.abs(blk).max(axis=(2, 3)))
        scales[:, :, t] = scale
        q = np.rint(blk / scale[:, :, None, None])
        codes[:, :, t * block:min(S, (t + 1) * block)] = np.clip(q, -QMAX, QMAX).astype(np.int8)
    return codes, scales


def quantize_qk(q, k, kmean=None):
    """Rules 1-5 applied to Q and K (fp64 arrays holding bf16 values, [B, H, S, D]).

    Returns a dict with k_mean [B,H,D] f32, q_codes, k_codes int8 [B,H,S,D],
    q_scale f32 [B,H,ceil(S/128)], k_scale f32 [B,H,ceil(S/64)].
    """
    q = np.asarray(q, dtype=np.float64)
    if kmean is None:
        kmean = k_channel_mean(k)
    qc, qs = quantize_blocks(q.astype(np.float32), Q_BLOCK)
    kc, ks = quantize_blocks(smooth_k(k, kmean), K_BLOCK)
    return {"k_mean": kmean, "q_codes": qc, "q_scale": qs, "k_codes": kc, "k_scale": ks}


def attention_int8(q_codes, q_scale, k_codes, k_scale, v, scale: float | None = None,
                   rows=None, q_block: int = Q_BLOCK, k_block: int = K_BLOCK) -> np.ndarray:
    """Attention on int8 codes (rule 6), fp64; rows selects query rows (default: all).

    q_codes, k_codes: int8 [B, H, S, D]; q_scale, k_scale: float32 per block; v: [B, H, S, Dv].
    """
    q_codes = np.asarray(q_codes)
    k_codes = np.asarray(k_codes)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = q_codes.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    sq_rows = np.asarray(q_scale, dtype=np.float64)[:, :, rows // q_block]
    sk_cols = np.repeat(np.asarray(k_scale, dtype=np.float64), k_block, axis=2)[:, :, :k_codes.shape[2]]
    out = np.empty((B, H, rows.size, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kc = np.ascontiguousarray(k_codes[b, h].astype(np.float64).T)
            for r0 in range(0, rows.size, 1024):
                r = rows[r0:r0 + 1024]
                dots = q_codes[b, h, r].astype(np.float64) @ kc
                s = dots * sq_rows[b, h, r0:r0 + 1024, None] * sk_cols[b, h][None, :] * scale
                w = np.exp(s - s.max(axis=1, keepdims=True))
                out[b, h, r0:r0 + 1024] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
    return out


def log_sum_exp_int8(q_codes, q_scale, k_codes, k_scale, scale: float | None = None,
                     q_block: int = Q_BLOCK, k_block: int = K_BLOCK) -> np.ndarray:
    """log sum_j exp(s_ij) of the int8-path scores (rule 6: s = codes . codes x scales x scale),
    fp64 [B, H, S] — the normaliser that goes with attention_int8."""
    q_codes = np.asarray(q_codes)
    k_codes = np.asarray(k_codes)
    B, H, S, D = q_codes.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.arange(S)
    sq_rows = np.asarray(q_scale, dtype=np.float64)[:, :, rows // q_block]
    sk_cols = np.repeat(np.asarray(k_scale, dtype=np.float64), k_block, axis=2)[:, :, :k_codes.shape[2]]
    out = np.empty((B, H, S), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kc = np.ascontiguousarray(k_codes[b, h].astype(np.float64).T)
            for r0 in range(0, S, 1024):
                r = rows[r0:r0 + 1024]
                dots = q_codes[b, h, r].astype(np.float64) @ kc
                sc = dots * sq_rows[b, h, r0:r0 + 1024, None] * sk_cols[b, h][None, :] * scale
                m = sc.max(axis=1)
                out[b, h, r0:r0 + 1024] = m + np.log(np.exp(sc - m[:, None]).sum(axis=1))
    return out


def probe_rows(S: int, n_rows: int) -> np.ndarray:
    """The query rows a quantization-error probe samples (this library's choice): with
    step = floor(S / n_rows), row i = floor(step / 2) + i * step, the middle row of the i-th of
    n_rows bins of step consecutive rows (the upper of the two middle rows when step is even;
    the last S - n_rows * step rows are never sampled)."""
    step = S // n_rows
    return step // 2 + np.arange(n_rows, dtype=np.int64) * step


def quant_probe_error(q, k, v, n_rows: int, scale: float | None = None):
    """Relative L2 error of the int8-QK output against exact attention on the sampled rows.

    The "TMAP image-to-video inference acceleration" page (section on preserving video quality)
    keeps some attention layers in full precision, chosen by the per-layer error of the
    quantized attention over the denoising steps; this is that error for one call:
    sqrt(sum |o_int8 - o|^2 / sum |o|^2) over the rows probe_rows(S, n_rows) of every (b, h)
    (o = exact attention, o_int8 = attention_int8 on this module's quantization), overall and
    per (b, h).  q, k, v: fp64 [B, H, S, D] holding bf16 values.  Returns (overall, [B, H])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, S, D = q.shape
    rows = probe_rows(S, n_rows)
    from .attention import attention_rows
    ref = quantize_qk(q, k)
    exact = attention_rows(q, k, v, rows, scale)
    quant = attention_int8(ref["q_codes"], ref["q_scale"], ref["k_codes"], ref["k_scale"], v,
                           scale, rows=rows)
    num = ((quant - exact) ** 2).sum(axis=(2, 3))
    den = (exact ** 2).sum(axis=(2, 3))
    return float(np.sqrt(num.sum() / den.sum())), np.sqrt(num / den)


# ---- fp8 (OCP e4m3) codes ---------------------------------------------------------------------
#
# The same steps with fp8 codes instead of int8 (this library's fp8 contract; the pages run
# their linear layers in fp8 and their attention in 8 bits):
#   scale = amax / 448 (IEEE fp32 division; 448 is the largest finite e4m3 value), 1.0 if
#   amax == 0; code = e4m3(clamp(fl32(x / scale), -448, 448)), rounded once to nearest even.
# e4m3 (OCP "E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 fraction bits; normal values
# (1 + m/8) 2^(e-7) for e = 1..15 (e = 15, m = 7 is NaN, so the largest is 448); subnormal
# values m/8 * 2^-6; no infinities.

E4M3_MAX = 448.0


def e4m3_value(codes) -> np.ndarray:
    """fp64 values of e4m3 codes (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _e4m3_table():
    vals = e4m3_value(np.arange(128, dtype=np.uint8))   # non-negative codes 0..127
    return vals[:127]                                    # drop the NaN code 0x7F


def e4m3_round(x) -> np.ndarray:
    """Round fp64 values with |x| <= 448 to the nearest e4m3 value (ties to the even code,
    i.e. the one with an even fraction field); returns uint8 codes.  As in any IEEE rounding
    the sign is kept, also when the result is zero: a negative value below half the smallest
    subnormal (and -0) gives -0, code 0x80."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~(np.abs(x) <= E4M3_MAX)):
        raise ValueError("e4m3_round takes finite values of magnitude <= 448")
    grid = _e4m3_table()                 # increasing, codes 0..126
    a = np.abs(x)
    hi = np.searchsorted(grid, a, side="left")        # first grid value >= a
    hi = np.minimum(hi, grid.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == grid[hi], hi, np.where(pick_hi, hi, lo)).astype(np.int64)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_blocks_fp8(x, block: int):
    """e4m3 codes (uint8 [B, H, S, D]) and per-block scales (float32 [B, H, nblk])."""
    x = np.asarray(x, dtype=np.float32)
    B, H, S, D = x.shape
    nblk = -(-S // block)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    codes = np.empty((B, H, S, D), dtype=np.uint8)
    for t in range(nblk):
        blk = x[:, :, t * block:min(S, (t + 1) * block)]
        amax = np.abs(blk).max(axis=(2, 3))
        scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
        scales[:, :, t] = scale
        q = np.clip(blk / scale[:, :, None, None], np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[:, :, t * block:min(S, (t + 1) * block)] = e4m3_round(q.astype(np.float64))
    return codes, scales


def quantize_qk_fp8(q, k, kmean=None):
    """quantize_qk with e4m3 codes: same K mean and smoothing, scale = amax / 448."""
    q = np.asarray(q, dtype=np.float64)
    if kmean is None:
        kmean = k_channel_mean(k)
    qc, qs = quantize_blocks_fp8(q.astype(np.float32), Q_BLOCK)
    kc, ks = quantize_blocks_fp8(smooth_k(k, kmean), K_BLOCK)
    return {"k_mean": kmean, "q_codes": qc, "q_scale": qs, "k_codes": kc, "k_scale": ks}


def attention_fp8(q_codes, q_scale, k_codes, k_scale, v, scale: float | None = None, rows=None):
    """Attention on e4m3 codes: s_ij = (sum_d q_id k_jd) * sq * sk * scale with the code values,
    then the exact softmax and PV, all in fp64 (as attention_int8)."""
    return attention_int8(e4m3_value(q_codes), q_scale, e4m3_value(k_codes), k_scale, v, scale,
                          rows=rows)


def log_sum_exp_fp8(q_codes, q_scale, k_codes, k_scale, scale: float | None = None):
    """log sum_j exp(s_ij) of the fp8-path scores, fp64 [B, H, S]."""
    return log_sum_exp_int8(e4m3_value(q_codes), q_scale, e4m3_value(k_codes), k_scale, scale)


# ---- fp8 for both products ---------------------------------------------------------------------
#
# The fp8 variant with V in e4m3 as well (PV on the fp8 matrix cores), this library's contract:
#   V: one scale per (b, h, channel) over all S tokens, scale_v = amax / 448 (1.0 if amax == 0),
#      code = e4m3(clamp(fl32(v / scale_v), -448, 448)), rounded once (as the Q / K codes).
#   o_i = sum_j p_ij * vq_jd * scale_v[d] / sum_j p_ij  with p the exact softmax weights of the
#      fp8 scores.  (The GPU rounds each weight to e4m3 at its running offset before the product
#      and normalises by the sum of those rounded weights; that rounding is not part of this
#      definition: it perturbs every weight by at most 2^-4 relative, and the parity tolerance
#      covers it.)

def quantize_v_fp8(v):
    """Per-(b, h, channel) e4m3 codes of V: (codes uint8 [B, H, S, D], scales float32 [B, H, D])."""
    x = np.asarray(v, dtype=np.float64).astype(np.float32)
    amax = np.abs(x).max(axis=2)                                            # [B, H, D]
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = np.clip(x / scale[:, :, None, :], np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_round(q.astype(np.float64)), scale


def attention_fp8_full(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale,
                       scale: float | None = None, rows=None):
    """Attention with fp8 scores (as attention_fp8) and fp8 V: the exact softmax of the scores
    applied to the dequantized V (codes times their channel scale), fp64."""
    vq = e4m3_value(v_codes) * np.asarray(v_scale, dtype=np.float64)[:, :, None, :]
    return attention_fp8(q_codes, q_scale, k_codes, k_scale, vq, scale, rows=rows)
