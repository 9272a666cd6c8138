"""First Block Cache: the per-step cache decision and the residual arithmetic around it.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix:

* "ParaAttention" page, First Block Cache section: the difference between the first transformer
  block's output residual at this denoising step and at the previous one stands in for the
  difference between model outputs; when it is small enough the previous step's residual is
  reused, i.e. the remaining blocks of the step are skipped.  FLUX's default threshold is 0.08.
* "Cache-DiT acceleration" page (vLLM-Omni user guide), DBCache parameters and configuration
  reference: ``residual_diff_threshold`` (default 0.24; larger caches more),
  ``max_warmup_steps`` (default 4: the first steps never use the cache),
  ``max_cached_steps`` (default -1 = no limit on cached steps) and
  ``max_continuous_cached_steps`` (default 3: a limit on consecutive cached steps).

Readings where the pages are silent (this library's contract):

1. The difference is the relative L1 distance of ``rel_l1`` (this package), rounded to fp32,
   and a step may use the cache only when ``diff < threshold`` (strict; both fp32).  A NaN
   difference never passes.
2. Steps are numbered from 0; step t is a warmup step when t < max_warmup_steps.
3. A step with no previous residual (the first computed step) computes.
4. max_cached_steps = M >= 0 allows at most M cached steps in the run; -1 is no limit.
   max_continuous_cached_steps = C >= 0 allows at most C cached steps in a row (the step after
   C of them computes; C = 0 never caches); -1 is no limit.
5. The previous residual a step compares against is the first-block residual of the latest
   step that computed (a cached step does not replace it).
6. Applying a residual, ``out = h + r``, and forming one, ``r = a - b``, round the exact result
   of the bf16 operands once to bf16 (nearest, ties to even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .rel_l1 import rel_l1


@dataclasses.dataclass(frozen=True)
class FBCacheConfig:
    residual_diff_threshold: float = 0.24
    max_warmup_steps: int = 4
    max_cached_steps: int = -1
    max_continuous_cached_steps: int = 3


@dataclasses.dataclass(frozen=True)
class FBCacheState:
    steps: int = 0              # steps decided so far
    cached_steps: int = 0       # of them, served from the cache
    continuous: int = 0         # cached steps since the latest computed step
    use_cache: bool = False     # decision of the latest step
    diff: float = math.nan      # difference of the latest step (NaN: no previous residual)


def fbcache_decide(state: FBCacheState, cfg: FBCacheConfig, diff) -> FBCacheState:
    """One step's decision (readings 1-4).  diff: the step's difference, or None when there is
    no previous residual.  Returns the new state; its use_cache is the decision."""
    d = math.nan if diff is None else float(np.float32(diff))
    thr = float(np.float32(cfg.residual_diff_threshold))
    use = True
    if state.steps < cfg.max_warmup_steps:
        use = False
    if diff is None or not (d < thr):
        use = False
    if cfg.max_cached_steps >= 0 and state.cached_steps >= cfg.max_cached_steps:
        use = False
    if cfg.max_continuous_cached_steps >= 0 and state.continuous >= cfg.max_continuous_cached_steps:
        use = False
    return FBCacheState(steps=state.steps + 1,
                        cached_steps=state.cached_steps + (1 if use else 0),
                        continuous=state.continuous + 1 if use else 0,
                        use_cache=use, diff=d)


def fbcache_run(residuals, cfg: FBCacheConfig):
    """Decisions over a sequence of first-block residuals (one per step), reading 5 for the
    reference residual.  Returns a list of states, one per step."""
    state, prev, out = FBCacheState(), None, []
    for r in residuals:
        state = fbcache_decide(state, cfg, None if prev is None else rel_l1(r, prev))
        if not state.use_cache:
            prev = r
        out.append(state)
    return out


# ---- residual arithmetic (reading 6) ---------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, fp32's exponent range), nearest with ties
    to even, overflow to inf; returns the uint16 bit patterns.

    Normal range: round the fp64 significand to 7 fraction bits (a carry may step the exponent),
    then the value is exact in fp32 and its upper half is the bf16 pattern.  Below 2^-126 bf16
    is fixed point with step 2^-133: round x * 2^133 to an integer."""
    x = np.asarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    keep_odd = (bits >> np.uint64(45)) & np.uint64(1)
    rounded = ((bits + np.uint64((1 << 44) - 1) + keep_odd) & ~np.uint64((1 << 45) - 1)).view(np.float64)
    tiny = np.abs(x) < 2.0 ** -126
    sub = np.rint(x * 2.0 ** 133) * 2.0 ** -133
    y = np.where(tiny, sub, rounded)
    y = np.where(np.isnan(x), np.nan, y)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _bf16_value(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def resid_add(a_bits, b_bits) -> np.ndarray:
    """bf16(a + b) for bf16 bit patterns.  The fp64 sum is exact unless the exponents differ by
    more than 45, where its one rounding is innocuous before the rounding to 8 bits (53 >= 2*8+2),
    so the result is the exact sum rounded once."""
    return bf16_round(_bf16_value(a_bits) + _bf16_value(b_bits))


def resid_sub(a_bits, b_bits) -> np.ndarray:
    """bf16(a - b) for bf16 bit patterns (as resid_add)."""
    return bf16_round(_bf16_value(a_bits) - _bf16_value(b_bits))
