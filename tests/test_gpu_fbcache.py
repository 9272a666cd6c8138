"""GPU tests of the First Block Cache calls (fbcache_decide, resid_add, resid_sub) against the
oracle (oracle/fbcache.py).

Bar: decisions and state counters exact; the stored difference equal to resid_rel_l1 on the
same tensors (same kernel) and within 1e-4 relative of the oracle's fp64 value; residual
add / subtract bit-exact (each value the exact result rounded once to bf16).  A decision
compares a floating-point difference with the threshold, so the sequences below keep every
difference at least 1% away from the threshold (asserted): there the GPU's and the oracle's
difference take the same side.
"""
import math
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

RL1_REL = 1e-4
MARGIN = 0.01


def announce(msg):
    print(f"[gpu-fbcache] {msg}", file=sys.stderr, flush=True)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return datagen.bf16_to_f64(bits)


# ---------------------------------------------------------------------------------------------
# residual add / subtract
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 7, 8, 9, 4095, (1 << 20) + 5])
def test_resid_add_sub_bit_exact(n):
    announce(f"resid_add / resid_sub n={n}")
    rng = np.random.default_rng(n)
    a = datagen.f64_to_bf16_bits(rng.standard_normal(n) * 2.0 ** rng.integers(-12, 13, n))
    b = datagen.f64_to_bf16_bits(rng.standard_normal(n) * 2.0 ** rng.integers(-12, 13, n))
    da, db = dev(a), dev(b)
    s, d = dta.resid_add(da, db), dta.resid_sub(da, db)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(s), oracle.resid_add(a, b))
    assert np.array_equal(host_bits(d), oracle.resid_sub(a, b))


def test_resid_add_sub_in_place_and_edge_values():
    announce("resid_add / resid_sub in place, wide exponent gaps, subnormal and overflowing sums")
    n = 1000
    rng = np.random.default_rng(5)
    a = datagen.f64_to_bf16_bits(rng.standard_normal(n) * 2.0 ** rng.integers(-60, 61, n))
    b = datagen.f64_to_bf16_bits(rng.standard_normal(n) * 2.0 ** rng.integers(-60, 61, n))
    # sums near the bottom of the range and at the top (overflow to inf)
    a[:4] = datagen.f64_to_bf16_bits(np.array([2.0 ** -130, -2.0 ** -128, 3.0e38, -3.0e38]))
    b[:4] = datagen.f64_to_bf16_bits(np.array([2.0 ** -131, 2.0 ** -127, 3.0e38, -3.0e38]))
    want_add, want_sub = oracle.resid_add(a, b), oracle.resid_sub(a, b)
    da, db = dev(a), dev(b)
    dta.resid_add(da, db, out=da)            # in place on a
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(da), want_add)
    da, db = dev(a), dev(b)
    dta.resid_sub(da, db, out=db)            # in place on b
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(db), want_sub)


def test_resid_add_longvideo_sampled():
    rows, cols = 118800, 3072
    announce(f"resid_add / resid_sub [{rows}, {cols}] (sampled elements)")
    a, b = datagen.residual_pair(rows, cols)
    da, db = dev(a), dev(b)
    s, d = dta.resid_add(da, db), dta.resid_sub(da, db)
    torch.cuda.synchronize()
    n = rows * cols
    idx = np.concatenate([np.arange(4096), np.arange(n - 4096, n),
                          np.random.default_rng(3).choice(n, 1 << 20, replace=False)])
    ti = torch.from_numpy(idx).cuda()
    sa = host_bits(s.view(-1).index_select(0, ti))
    sd = host_bits(d.view(-1).index_select(0, ti))
    a1, b1 = a.reshape(-1)[idx], b.reshape(-1)[idx]
    assert np.array_equal(sa, oracle.resid_add(a1, b1))
    assert np.array_equal(sd, oracle.resid_sub(a1, b1))


# ---------------------------------------------------------------------------------------------
# the cache decision
# ---------------------------------------------------------------------------------------------

def _state(st):
    return dta.fbcache_state_values(st)


def test_decide_reference_rule_closed_form():
    """r_t = c_t * base (exact in bf16), scales 1, 17/16, 18/16, 19/16, threshold 0.1: the
    differences are exactly 1/16, 1/8 (against step 0: step 1 was cached) and 1/18."""
    announce("fbcache_decide closed-form sequence")
    base = np.array([0.5, -0.75, 1.5, -3.5, 1.75, -0.875, 2.5, 3.0] * 1000)
    res = [dev(datagen.f64_to_bf16_bits(c * base)) for c in (1.0, 17 / 16, 18 / 16, 19 / 16)]
    assert all(np.array_equal(f64(host_bits(r)), c * base)
               for r, c in zip(res, (1.0, 17 / 16, 18 / 16, 19 / 16)))
    cfg = dta.FBCacheConfig(0.1, 0, -1, -1)
    st = dta.fbcache_state("cuda")
    ref, got = None, []
    for r in res:
        dta.fbcache_decide(r, ref, st, cfg)
        v = _state(st)
        got.append(v)
        if not v["use_cache"]:
            ref = r
    assert [v["use_cache"] for v in got] == [0, 1, 0, 1]
    assert math.isnan(got[0]["diff"])
    assert [v["diff"] for v in got[1:]] == [float(np.float32(x)) for x in (1 / 16, 1 / 8, 1 / 18)]
    assert got[-1]["steps"] == 4 and got[-1]["cached_steps"] == 2
    assert got[-1]["continuous_cached_steps"] == 1


def test_decide_special_differences():
    announce("fbcache_decide: zero reference, NaN residual")
    n = 4099
    z = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    x = dev(datagen.normal_bf16((n,), 9, 0))
    xn = x.clone()
    xn[17] = float("nan")
    cfg = dta.FBCacheConfig(0.5, 0, -1, -1)
    st = dta.fbcache_state("cuda")
    dta.fbcache_decide(z, None, st, cfg)
    assert _state(st)["use_cache"] == 0
    dta.fbcache_decide(z, z, st, cfg)                  # 0 / 0 -> 0: reuse
    v = _state(st)
    assert v["use_cache"] == 1 and v["diff"] == 0.0
    dta.fbcache_decide(x, z, st, cfg)                  # x / 0 -> inf: compute
    v = _state(st)
    assert v["use_cache"] == 0 and v["diff"] == math.inf
    dta.fbcache_decide(xn, x, st, cfg)                 # NaN: compute
    v = _state(st)
    assert v["use_cache"] == 0 and math.isnan(v["diff"])
    assert v["steps"] == 4 and v["cached_steps"] == 1 and v["continuous_cached_steps"] == 0


CONFIGS = {
    "cache_dit_defaults": (0.24, 4, -1, 3),
    "tight_threshold": (0.08, 0, -1, -1),
    "total_cap": (0.095, 1, 2, -1),
    "runs_of_two": (0.2, 2, -1, 2),
    "never": (0.0, 0, -1, -1),
}
DRIFT = [0.02, 0.02, 0.02, 0.02, 0.3, 0.02, 0.02, 0.02, 0.02, 0.02, 0.02, 0.02, 0.3, 0.02]


@pytest.fixture(scope="module")
def run_steps():
    seq = datagen.hidden_state_steps(len(DRIFT), 256, 3072, drift=DRIFT)
    return seq


@pytest.mark.parametrize("name", list(CONFIGS))
def test_decide_sequence_matches_oracle(name, run_steps):
    """A denoising run driven through the library (residuals with resid_sub, decision with
    fbcache_decide, cached steps with resid_add) against the same run in the oracle: decisions,
    counters and every step's output bit-exact."""
    thr, warm, cap, cont = CONFIGS[name]
    announce(f"fbcache run '{name}': threshold {thr}, warmup {warm}, cap {cap}, in a row {cont}")
    ocfg = oracle.FBCacheConfig(thr, warm, cap, cont)
    # oracle run
    ostate, oref, orest, oout, ostates, odiffs = oracle.FBCacheState(), None, None, [], [], []
    for h0, h1, hn in run_steps:
        r1 = oracle.resid_sub(h1, h0)
        d = None if oref is None else oracle.rel_l1(f64(r1), f64(oref))
        ostate = oracle.fbcache_decide(ostate, ocfg, d)
        if d is not None and thr > 0:
            assert abs(d - thr) >= MARGIN * thr, f"difference {d} too close to threshold {thr}"
        if ostate.use_cache:
            oout.append(oracle.resid_add(h1, orest))
        else:
            orest = oracle.resid_sub(hn, h1)
            oout.append(hn)
            oref = r1
        ostates.append(ostate)
        odiffs.append(d)
    # library run
    cfg = dta.FBCacheConfig(thr, warm, cap, cont)
    st = dta.fbcache_state("cuda")
    ref = rest = None
    bufs = [torch.empty(256 * 3072, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    cur = 0
    for t, (h0, h1, hn) in enumerate(run_steps):
        g0, g1 = dev(h0).view(-1), dev(h1).view(-1)
        r1 = dta.resid_sub(g1, g0, out=bufs[cur])
        dta.fbcache_decide(r1, ref, st, cfg)
        v = _state(st)
        if ref is not None:
            want = dta.resid_rel_l1(r1, ref)
            assert v["diff"] == float(want.item()), t
            assert abs(v["diff"] - odiffs[t]) <= RL1_REL * odiffs[t], (t, v["diff"], odiffs[t])
        assert v["use_cache"] == int(ostates[t].use_cache), (name, t, v, ostates[t])
        assert (v["steps"], v["cached_steps"], v["continuous_cached_steps"]) == \
            (ostates[t].steps, ostates[t].cached_steps, ostates[t].continuous), (name, t)
        if v["use_cache"]:
            out = dta.resid_add(g1, rest)
        else:
            gn = dev(hn).view(-1)
            rest = dta.resid_sub(gn, g1)
            out = gn
            ref = r1
            cur ^= 1          # the reference keeps its buffer; the next residual takes the other
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), oout[t].reshape(-1)), (name, t)
    decisions = [int(s.use_cache) for s in ostates]
    announce(f"  decisions {decisions}")
    if name != "never":
        assert any(decisions) and not all(decisions)
