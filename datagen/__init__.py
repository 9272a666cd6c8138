"""Seeded synthetic inputs for DiT attention and the first-block-cache reduction.

This module only draws random numbers and rounds them to the input dtype (bf16).  It holds
none of the attention, quantization or reduction arithmetic, so both the fp64 oracle and the
HIP path can take their inputs from it without sharing any of the method's code.

Every tensor is drawn from its own numpy PCG64 stream, keyed by
``SeedSequence([workload_id, tag, b, h])`` (tags below), as fp64 normals, shifted / scaled in
fp64, rounded to fp32 (round-to-nearest) and then to bf16 (round-to-nearest-even on the fp32
bits).  The result is returned as ``uint16`` bf16 bit patterns; ``bf16_to_f64`` widens them
exactly.

Workload shapes follow the sequence lengths the pages describe:

* ``tiny``: B=1, H=2, S=256, D=64, plain N(0,1) for Q, K, V.
* ``image``: a 1024x1024 single-stream DiT (64x64 latent patches = 4096 image tokens + 512 text
  tokens, S=4608, H=24, D=128); the "Flash Attention 2 for Z-Image S3-DiT" page describes
  this single-stream concatenation of text and image tokens at >4000 tokens, and the
  ParaAttention page runs FLUX.1-dev at 1024x1024.
* ``video``: a 704x1280x49-frame latent (22x40 patches x 13 latent frames = 11440 tokens),
  B=2 for the conditional and unconditional pass (Wan2.2 TI2V example with guidance on the
  "Diffusion Attention Backends" page).
* ``longvideo``: a 720p 129-frame latent (45x80 patches x 33 latent frames = 118800 tokens),
  the HunyuanVideo run of the ParaAttention page.

For ``image``, ``video`` and ``longvideo`` each K channel gets an offset c[h, d] ~ N(0, 2)
(variance 2), shared over batch and tokens, to mimic per-channel outliers.
"""
from __future__ import annotations

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_KOFF, TAG_RL1_B, TAG_RL1_NOISE = 0, 1, 2, 3, 4, 5
TAG_FB_H0, TAG_FB_STEP, TAG_FB_FIRST, TAG_FB_REST = 6, 7, 8, 9

# name -> (workload_id, B, H, S, D, K-offset variance)
WORKLOADS = {
    "tiny": (0, 1, 2, 256, 64, 0.0),
    "image": (1, 1, 24, 4608, 128, 2.0),
    "video": (3, 2, 24, 11440, 128, 2.0),
    "longvideo": (4, 1, 24, 118800, 128, 2.0),
}

# hidden size of the first-block residual (24 heads x 128)
RL1_HIDDEN = 3072
RL1_NOISE = 0.05


def _stream(workload_id: int, tag: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, tag, b, h])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even), returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """fp64 -> fp32 (round-to-nearest) -> bf16 (round-to-nearest-even)."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_to_f32(bits).astype(np.float64)


def k_offsets(workload_id: int, H: int, D: int, var: float) -> np.ndarray:
    """Per-(head, channel) K offsets c[h, d] ~ N(0, var), fp64."""
    if var == 0.0:
        return np.zeros((H, D))
    return np.sqrt(var) * _stream(workload_id, TAG_KOFF).standard_normal((H, D))


def qkv_head(workload_id: int, b: int, h: int, S: int, D: int, koff_row=None):
    """Q, K, V of one (batch, head) as bf16 bits [S, D] each."""
    q = f64_to_bf16_bits(_stream(workload_id, TAG_Q, b, h).standard_normal((S, D)))
    kz = _stream(workload_id, TAG_K, b, h).standard_normal((S, D))
    if koff_row is not None:
        kz = kz + koff_row[None, :]
    k = f64_to_bf16_bits(kz)
    v = f64_to_bf16_bits(_stream(workload_id, TAG_V, b, h).standard_normal((S, D)))
    return q, k, v


def attention_inputs(name: str):
    """Q, K, V bf16 bits [B, H, S, D] for a named workload."""
    wid, B, H, S, D, var = WORKLOADS[name]
    off = k_offsets(wid, H, D, var)
    q = np.empty((B, H, S, D), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            q[b, h], k[b, h], v[b, h] = qkv_head(wid, b, h, S, D, off[h] if var else None)
    return q, k, v


def with_zero_k_channel(k_bits: np.ndarray, head: int = 0, channel: int = 0) -> np.ndarray:
    """Copy of K with one channel of one head set to +0.0 for every batch and token."""
    out = k_bits.copy()
    out[:, head, :, channel] = 0
    return out


def normal_bf16(shape, workload_id: int, tag: int, b: int = 0, h: int = 0) -> np.ndarray:
    """N(0, 1) values rounded to bf16 bits, from the stream (workload_id, tag, b, h)."""
    return f64_to_bf16_bits(_stream(workload_id, tag, b, h).standard_normal(shape))


def residual_pair(rows: int, cols: int = RL1_HIDDEN, workload_id: int = 4, noise: float = RL1_NOISE):
    """First-block residuals (a, b), bf16 bits [rows, cols]: b ~ N(0, 1), a = b + noise * N(0, 1)."""
    b = f64_to_bf16_bits(_stream(workload_id, TAG_RL1_B).standard_normal((rows, cols)))
    n = _stream(workload_id, TAG_RL1_NOISE).standard_normal((rows, cols))
    a = f64_to_bf16_bits(bf16_to_f64(b) + noise * n)
    return a, b


def hidden_state_steps(steps: int, rows: int, cols: int = RL1_HIDDEN, drift=None,
                       workload_id: int = 5):
    """Synthetic hidden states of a denoising run, as bf16 bits [rows, cols] per step:
    h0 (the step's input), h1 (after the first block) and hN (after the last block).

    h0 and the first block's own contribution (0.5 * N(0, 1) at step 0) are random walks over
    the steps: step t moves each by drift[t] * N(0, 1).  The remaining blocks add a fresh
    N(0, 1).  Small drift makes consecutive first-block residuals close, and the distance to
    an older step grows with the number of steps in between."""
    drift = [0.02] * steps if drift is None else list(drift)
    g0 = _stream(workload_id, TAG_FB_H0)
    first = 0.5 * _stream(workload_id, TAG_FB_FIRST).standard_normal((rows, cols))
    h = g0.standard_normal((rows, cols))
    out = []
    for t in range(steps):
        gs = _stream(workload_id, TAG_FB_STEP, t)
        h = h + drift[t] * gs.standard_normal((rows, cols))
        first = first + drift[t] * gs.standard_normal((rows, cols))
        rest = _stream(workload_id, TAG_FB_REST, t).standard_normal((rows, cols))
        h0 = f64_to_bf16_bits(h)
        h1 = f64_to_bf16_bits(bf16_to_f64(h0) + first)
        hn = f64_to_bf16_bits(bf16_to_f64(h1) + rest)
        out.append((h0, h1, hn))
    return out


def sample_rows(S: int, n_random: int, seed: int, edge: int = 64) -> np.ndarray:
    """Sorted distinct row indices: the first and last `edge` rows plus `n_random` seeded ones."""
    edge = min(edge, S)
    fixed = set(range(edge)) | set(range(S - edge, S))
    rest = np.setdiff1d(np.arange(S), np.fromiter(fixed, dtype=np.int64))
    g = _stream(seed, 99)
    pick = g.choice(rest, size=min(n_random, rest.size), replace=False) if rest.size else []
    return np.array(sorted(fixed | set(int(i) for i in pick)), dtype=np.int64)
