"""Pins of the First Block Cache oracle (oracle/fbcache.py): hand-worked decision sequences,
closed-form residual sequences, exact rational rounding and torch's own bf16 arithmetic."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle.fbcache as fb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _diff(x):
    if x is None:
        return None
    return float(x)  # also "inf" and "nan"


def test_decisions_golden_worked_sequences():
    cases = json.load(open(os.path.join(GOLDEN, "fbcache_worked.json")))["cases"]
    for case in cases:
        cfg = fb.FBCacheConfig(**case["config"])
        st = fb.FBCacheState()
        got = []
        for d in case["diffs"]:
            st = fb.fbcache_decide(st, cfg, _diff(d))
            got.append(int(st.use_cache))
        assert got == case["use_cache"], case["name"]
        assert st.steps == len(case["diffs"])
        assert st.cached_steps == sum(case["use_cache"])


def test_state_counters_and_stored_difference():
    cfg = fb.FBCacheConfig(residual_diff_threshold=0.5, max_warmup_steps=0,
                           max_cached_steps=-1, max_continuous_cached_steps=-1)
    st = fb.fbcache_decide(fb.FBCacheState(), cfg, None)
    assert not st.use_cache and math.isnan(st.diff) and st.steps == 1
    st = fb.fbcache_decide(st, cfg, 0.1)
    assert st.use_cache and st.continuous == 1 and st.cached_steps == 1
    assert st.diff == float(np.float32(0.1))          # the fp32 difference is kept
    st = fb.fbcache_decide(st, cfg, 0.7)
    assert not st.use_cache and st.continuous == 0 and st.cached_steps == 1


def test_threshold_compared_in_fp32():
    # 0.1 is not exact in fp32; a difference equal to fp32(0.1) does not pass, one ulp below does
    cfg = fb.FBCacheConfig(residual_diff_threshold=0.1, max_warmup_steps=0,
                           max_cached_steps=-1, max_continuous_cached_steps=-1)
    t32 = np.float32(0.1)
    below = np.nextafter(t32, np.float32(0))
    st = fb.fbcache_decide(fb.FBCacheState(steps=1), cfg, float(t32))
    assert not st.use_cache
    st = fb.fbcache_decide(fb.FBCacheState(steps=1), cfg, float(below))
    assert st.use_cache


def _scaled_sequence(scales):
    """r_t = c_t * base with every product exact in bf16 (3-bit base values, 5-bit scales), so
    rel_l1(r_a, r_b) = |c_a - c_b| / |c_b| exactly."""
    base = np.array([0.5, -0.75, 1.5, -3.5, 1.75, -0.875, 2.5, 3.0] * 8)
    return [c * base for c in scales]


def test_reference_residual_is_the_latest_computed_step():
    # scales 1, 17/16, 18/16, 19/16 with threshold 0.1:
    #   step 1: |17/16 - 1| / 1 = 1/16 -> cached; the reference stays at step 0
    #   step 2: |18/16 - 1| / 1 = 1/8  -> computes; the reference becomes step 2
    #   step 3: (1/16) / (18/16) = 1/18 -> cached
    # (had step 1 replaced the reference, step 2 would see 1/17 and be cached)
    cfg = fb.FBCacheConfig(residual_diff_threshold=0.1, max_warmup_steps=0,
                           max_cached_steps=-1, max_continuous_cached_steps=-1)
    states = fb.fbcache_run(_scaled_sequence([1.0, 17 / 16, 18 / 16, 19 / 16]), cfg)
    assert [int(s.use_cache) for s in states] == [0, 1, 0, 1]
    assert math.isnan(states[0].diff)
    assert states[1].diff == float(np.float32(1 / 16))
    assert states[2].diff == float(np.float32(1 / 8))
    assert states[3].diff == float(np.float32(1 / 18))


# ---- rounding to bf16 -----------------------------------------------------------------------

def _exact_bf16(fr: Fraction) -> float:
    """Round a rational to bf16 by definition: 8 significant bits above 2^-126, a fixed step of
    2^-133 below, nearest with ties to even, overflow to inf."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 7)
    n, rem = divmod(a / quantum, 1)
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def _bits_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_bf16_round_matches_exact_rational_rounding():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.integers(-5, 6, 300),
        # exact midpoints between neighbouring bf16 values, and just off them
        (np.arange(256, 512) + 0.5) * 2.0 ** -8, (np.arange(256, 512) + 0.5) * 2.0 ** -8 + 2.0 ** -40,
        np.array([3.4e38, 3.3961776e38, 3.3961775e38, 1e39, -1e39, 2.0 ** -130 * 1.3,
                  2.0 ** -133 * 0.5, 2.0 ** -133 * 1.5, 2.0 ** -133 * 2.5, 2.0 ** -126 * 0.999999]),
    ])
    got = _bits_value(fb.bf16_round(x))
    for xi, gi in zip(x, got):
        ref = _exact_bf16(Fraction(float(xi)))
        assert gi == ref or (math.isinf(ref) and gi == ref), (xi, gi, ref)


def test_bf16_round_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)).astype(np.float32)
    x[:4] = [np.inf, -np.inf, 0.0, -0.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fb.bf16_round(x.astype(np.float64)), ref)
    nan_bits = fb.bf16_round(np.array([np.nan]))
    assert np.isnan(_bits_value(nan_bits)[0])


def _rand_bf16_bits(rng, n, spread):
    v = (rng.standard_normal(n) * 2.0 ** rng.integers(-spread, spread + 1, n)).astype(np.float32)
    return (v.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def test_resid_add_sub_match_exact_rational_arithmetic():
    rng = np.random.default_rng(13)
    a = _rand_bf16_bits(rng, 400, 60)   # exponent gaps up to 120: beyond fp64's 53 bits too
    b = _rand_bf16_bits(rng, 400, 60)
    s, d = fb.resid_add(a, b), fb.resid_sub(a, b)
    av, bv = _bits_value(a), _bits_value(b)
    for i in range(a.size):
        fa, fb_ = Fraction(float(av[i])), Fraction(float(bv[i]))
        assert _bits_value(s[i:i + 1])[0] == _exact_bf16(fa + fb_)
        assert _bits_value(d[i:i + 1])[0] == _exact_bf16(fa - fb_)


def test_resid_add_sub_match_torch_bf16_arithmetic():
    # torch adds bf16 tensors in fp32 and rounds once to bf16; rounding the exact sum to fp32
    # first is innocuous (24 >= 2*8+2 bits), so torch's result is the exact sum rounded once
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    a = _rand_bf16_bits(rng, 50000, 20)
    b = _rand_bf16_bits(rng, 50000, 20)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    assert np.array_equal(fb.resid_add(a, b), (ta + tb).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(fb.resid_sub(a, b), (ta - tb).view(torch.int16).numpy().view(np.uint16))


def test_apply_after_store_recovers_the_output_when_exact():
    # h + (f - h) == f whenever f - h is exact in bf16 (same exponent, values on a coarse grid)
    rng = np.random.default_rng(15)
    h = (rng.integers(-64, 64, 1000) / 16.0 + 8.0).astype(np.float32)
    f = (rng.integers(-64, 64, 1000) / 16.0 + 8.0).astype(np.float32)
    hb = (h.view(np.uint32) >> 16).astype(np.uint16)
    fb_bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    r = fb.resid_sub(fb_bits, hb)
    assert np.array_equal(fb.resid_add(hb, r), fb_bits)
