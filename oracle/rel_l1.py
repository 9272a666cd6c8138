"""Relative L1 distance of two residual tensors (test infrastructure only).

The "ParaAttention" page (section on First Block Cache) gates reuse of cached transformer
residuals on the difference between the first block's output residual at this step and at
the previous one: when the difference is small enough the remaining blocks are skipped.  The
page names the quantity, not its formula; this library reads it as the relative L1 distance

    r = mean |a - b| / mean |b| = sum |a - b| / sum |b|

with b the reference (previous) residual.  If sum |b| = 0: r = 0 when a == b everywhere,
otherwise +inf.  Computed in fp64; a - b of two bf16 values is exact in fp64.
"""
from __future__ import annotations

import numpy as np


def rel_l1(a, b) -> float:
    """sum|a - b| / sum|b| in fp64 over all elements of equally shaped arrays."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    num = np.abs(a - b).sum()
    den = np.abs(b).sum()
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
