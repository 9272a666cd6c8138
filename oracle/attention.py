"""Exact multi-head attention forward in fp64 (test infrastructure only).

What is computed: for every batch b, head h and query row i,

    s_j   = scale * sum_d q[i, d] * k[j, d]        (all keys j: non-causal, no mask)
    w_j   = exp(s_j - max_j s_j)
    o[i]  = sum_j w_j * v[j] / sum_j w_j

i.e. O = softmax(Q K^T * scale) V with the softmax over the key axis.  This is the operation
that the "Diffusion Attention Backends" page (vLLM-Omni, Overview and Backend Options) lets a
DiT swap between FlashAttention, torch scaled_dot_product_attention and SageAttention, and
that the "Flash Attention 2 for Z-Image S3-DiT" page (hotdry blog, method paragraph) computes
blockwise in on-chip memory without changing the result.  The scale is an argument; the
default of scaled_dot_product_attention, 1/sqrt(D), is what callers pass.

Subtracting the row maximum before exp changes nothing mathematically (the factor cancels in
the ratio) and keeps exp from overflowing.  Output rows are independent, so the loop over
query-row chunks below only bounds memory; it does not reorder any row's arithmetic.

The log-sum-exp of a row, lse_i = log sum_j exp(s_j), is the log of that ratio's denominator.
It is what lets results over disjoint key sets be merged exactly,

    lse = log(exp(lse_A) + exp(lse_B)),   o = exp(lse_A - lse) o_A + exp(lse_B - lse) o_B,

which is how a sequence split over devices (the ring dimension of the "ParaAttention" page's
context-parallel mesh, Context Parallelism section) combines its partial attention outputs.
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 1024


def _head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    kt = np.ascontiguousarray(k.T)
    for r0 in range(0, q.shape[0], _ROW_CHUNK):
        s = (q[r0:r0 + _ROW_CHUNK] @ kt) * scale
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[r0:r0 + _ROW_CHUNK] = (w @ v) / w.sum(axis=1, keepdims=True)
    return out


def attention(q, k, v, scale: float | None = None) -> np.ndarray:
    """softmax(q k^T * scale) v over [B, H, S, D] fp64 arrays; returns fp64 [B, H, Sq, Dv].

    q: [B, H, Sq, D]; k: [B, H, Sk, D]; v: [B, H, Sk, Dv].  scale defaults to 1/sqrt(D).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Sq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, H, Sq, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = _head(q[b, h], k[b, h], v[b, h], scale)
    return out


def attention_rows(q, k, v, rows, scale: float | None = None) -> np.ndarray:
    """Exact attention for the query rows `rows` only (same keys and values): [B, H, len(rows), Dv].

    Exact for those rows because each output row depends only on its own query row.
    """
    q = np.asarray(q, dtype=np.float64)
    return attention(q[:, :, np.asarray(rows)], k, v, scale)


def log_sum_exp(q, k, scale: float | None = None) -> np.ndarray:
    """lse[b, h, i] = log sum_j exp(scale * q_i . k_j) over all keys, fp64 [B, H, Sq].

    q: [B, H, Sq, D]; k: [B, H, Sk, D].  Computed as m + log(sum_j exp(s_j - m)), m = max_j s_j.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, Sq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kt = np.ascontiguousarray(k[b, h].T)
            for r0 in range(0, Sq, _ROW_CHUNK):
                sc = (q[b, h, r0:r0 + _ROW_CHUNK] @ kt) * scale
                m = sc.max(axis=1)
                out[b, h, r0:r0 + _ROW_CHUNK] = m + np.log(np.exp(sc - m[:, None]).sum(axis=1))
    return out
