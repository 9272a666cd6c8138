"""Pins for the fp64 oracle: brute force, closed forms, invariants, worked examples.

These run on the CPU only and check the oracle against facts fixed by the mathematics or
worked by hand, so a plausible slip in it (a dropped term, a wrong sign or index, a transposed
operand, a wrong block mapping, a non-IEEE rounding) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf(x):
    return datagen.bf16_to_f64(datagen.f64_to_bf16_bits(x))


# ---------------------------------------------------------------------------------------------
# exact attention
# ---------------------------------------------------------------------------------------------

def _brute_attention(q, k, v, scale):
    """Pure-Python loops, no max subtraction: only for tiny, small-valued inputs."""
    out = []
    for qi in q:
        e = [math.exp(scale * sum(a * b for a, b in zip(qi, kj))) for kj in k]
        z = sum(e)
        out.append([sum(e[j] * v[j][d] for j in range(len(k))) / z for d in range(len(v[0]))])
    return np.array(out)


@pytest.mark.parametrize("S,D,Dv", [(1, 1, 1), (2, 4, 3), (3, 8, 8), (5, 2, 7), (17, 16, 16)])
def test_attention_brute_force(S, D, Dv):
    rng = np.random.default_rng(S * 100 + D)
    q = rng.standard_normal((1, 1, S + 2, D))
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, Dv))
    scale = 1.0 / math.sqrt(D)
    got = oracle.attention(q, k, v)[0, 0]
    ref = _brute_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_attention_golden_worked_examples():
    for case in _load("attention_worked.json")["cases"]:
        q = np.array(case["q"])[None, None]
        k = np.array(case["k"])[None, None]
        v = np.array(case["v"])[None, None]
        got = oracle.attention(q, k, v, case["scale"])[0, 0]
        np.testing.assert_allclose(got, np.array(case["o"]), rtol=0, atol=case["tol"],
                                   err_msg=case["name"])


def test_single_key_returns_v():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((2, 3, n, 8)) for n in (5, 1, 1))
    got = oracle.attention(q, k, v)
    np.testing.assert_array_equal(got, np.broadcast_to(v, got.shape))


def test_two_keys_sigmoid_closed_form():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 6, 4))
    k = rng.standard_normal((1, 1, 2, 4))
    v = rng.standard_normal((1, 1, 2, 3))
    sc = 0.37
    got = oracle.attention(q, k, v, sc)[0, 0]
    s = sc * q[0, 0] @ k[0, 0].T
    w1 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    ref = w1[:, None] * v[0, 0, 0] + (1 - w1)[:, None] * v[0, 0, 1]
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_zero_query_gives_mean_of_v():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, 2, 37, 16)) * 5
    v = rng.standard_normal((2, 2, 37, 16))
    q = np.zeros((2, 2, 9, 16))
    got = oracle.attention(q, k, v)
    ref = np.broadcast_to(v.mean(axis=2, keepdims=True), got.shape)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-15)


def test_identical_value_rows_pass_through():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, 11, 8))
    k = rng.standard_normal((1, 2, 29, 8)) * 3
    row = rng.standard_normal(8)
    v = np.broadcast_to(row, (1, 2, 29, 8)).copy()
    got = oracle.attention(q, k, v)
    np.testing.assert_allclose(got, np.broadcast_to(row, got.shape), rtol=1e-14, atol=1e-15)


def test_joint_key_value_permutation_invariance():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 13, 8))
    k = rng.standard_normal((1, 2, 41, 8))
    v = rng.standard_normal((1, 2, 41, 5))
    perm = rng.permutation(41)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k[:, :, perm], v[:, :, perm])
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    # permuting only the values must change the result (a transposed / mis-indexed V would not)
    c = oracle.attention(q, k, v[:, :, perm])
    assert np.abs(a - c).max() > 1e-3


def test_key_channel_offset_invariance_exact():
    # q, k on a 1/16 grid, integer offsets, scale 1/4: every product, sum and shift is exact
    rng = np.random.default_rng(6)
    D = 16
    q = rng.integers(-64, 65, (1, 2, 10, D)) / 16.0
    k = rng.integers(-64, 65, (1, 2, 33, D)) / 16.0
    v = rng.standard_normal((1, 2, 33, D))
    c = rng.integers(-3, 4, (1, 2, 1, D)).astype(np.float64)
    a = oracle.attention(q, k, v)
    b = oracle.attention(q, k + c, v)
    np.testing.assert_array_equal(a, b)


def test_convex_combination_bounds():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 3, 20, 8)) * 4
    k = rng.standard_normal((1, 3, 50, 8))
    v = rng.standard_normal((1, 3, 50, 8))
    o = oracle.attention(q, k, v)
    lo = v.min(axis=2, keepdims=True) - 1e-14
    hi = v.max(axis=2, keepdims=True) + 1e-14
    assert np.all(o >= lo) and np.all(o <= hi)


def test_dominant_logit_selects_its_value_row_without_overflow():
    q = np.zeros((1, 1, 1, 4)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 6, 4)); k[0, 0, 3, 0] = 2000.0; k[0, 0, 1, 0] = 1000.0
    v = np.arange(24, dtype=np.float64).reshape(1, 1, 6, 4)
    o = oracle.attention(q, k, v, 1.0)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 3])


def test_against_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 3, 40, 32))
    k = rng.standard_normal((2, 3, 57, 32))
    v = rng.standard_normal((2, 3, 57, 24))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(oracle.attention(q, k, v), ref, rtol=1e-11, atol=1e-12)


def test_lse_brute_force_and_single_key():
    rng = np.random.default_rng(31)
    q, k = rng.standard_normal((1, 2, 4, 6)), rng.standard_normal((1, 2, 7, 6))
    sc = 0.41
    got = oracle.log_sum_exp(q, k, sc)
    for h in range(2):
        for i in range(4):
            z = sum(math.exp(sc * sum(a * b for a, b in zip(q[0, h, i], kj))) for kj in k[0, h])
            assert abs(got[0, h, i] - math.log(z)) < 1e-12
    # one key: the normaliser is exp(s), lse = s exactly up to rounding of the dot product
    k1 = k[:, :, :1]
    np.testing.assert_allclose(oracle.log_sum_exp(q, k1, sc)[..., None],
                               sc * q @ np.swapaxes(k1, -1, -2), rtol=0, atol=1e-13)


def test_lse_matches_scipy_logsumexp_and_survives_huge_scores():
    from scipy.special import logsumexp
    rng = np.random.default_rng(32)
    q, k = rng.standard_normal((2, 2, 9, 16)), rng.standard_normal((2, 2, 40, 16))
    s = (q @ np.swapaxes(k, -1, -2)) * 0.25
    np.testing.assert_allclose(oracle.log_sum_exp(q, k, 0.25), logsumexp(s, axis=-1),
                               rtol=1e-13, atol=1e-13)
    # scores near 2000 (exp overflows without the max shift): lse = 2000 + log(#equal maxima)
    k2 = np.zeros((1, 1, 3, 1)); k2[0, 0, :, 0] = [2000.0, 2000.0, 0.0]
    q2 = np.ones((1, 1, 1, 1))
    assert abs(oracle.log_sum_exp(q2, k2, 1.0)[0, 0, 0] - (2000.0 + math.log(2.0))) < 1e-12


def test_lse_merges_attention_over_disjoint_key_sets():
    # the property a sequence split over devices relies on: results over key halves A and B
    # combine into the full result through their log-sum-exps
    rng = np.random.default_rng(33)
    q = rng.standard_normal((1, 3, 11, 8))
    k = rng.standard_normal((1, 3, 30, 8)) * 2
    v = rng.standard_normal((1, 3, 30, 5))
    ka, kb, va, vb = k[:, :, :13], k[:, :, 13:], v[:, :, :13], v[:, :, 13:]
    la, lb = oracle.log_sum_exp(q, ka), oracle.log_sum_exp(q, kb)
    oa, ob = oracle.attention(q, ka, va), oracle.attention(q, kb, vb)
    lse = np.logaddexp(la, lb)
    np.testing.assert_allclose(lse, oracle.log_sum_exp(q, k), rtol=1e-13, atol=1e-13)
    merged = np.exp(la - lse)[..., None] * oa + np.exp(lb - lse)[..., None] * ob
    np.testing.assert_allclose(merged, oracle.attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_lse_shifts_with_a_common_score_offset():
    # adding u to every key with q . u = c for one query row shifts that row's lse by scale * c
    rng = np.random.default_rng(34)
    q = rng.standard_normal((1, 1, 1, 8))
    k = rng.standard_normal((1, 1, 25, 8))
    u = q[0, 0, 0] * (3.0 / float(q[0, 0, 0] @ q[0, 0, 0]))   # q . u = 3
    got = oracle.log_sum_exp(q, k + u, 0.5) - oracle.log_sum_exp(q, k, 0.5)
    assert abs(got[0, 0, 0] - 1.5) < 1e-12


def test_int8_lse_reduces_to_exact_lse_when_codes_are_the_values():
    # integer Q, K on the code grid with unit scales: the int8 normaliser equals the exact one
    rng = np.random.default_rng(35)
    qc = rng.integers(-127, 128, (1, 2, 130, 32)).astype(np.int8)
    kc = rng.integers(-127, 128, (1, 2, 70, 32)).astype(np.int8)
    qs = np.ones((1, 2, 2), np.float32)
    ks = np.ones((1, 2, 2), np.float32)
    sc = 1.0 / 4096
    got = oracle.log_sum_exp_int8(qc, qs, kc, ks, sc)
    np.testing.assert_allclose(got, oracle.log_sum_exp(qc.astype(np.float64), kc.astype(np.float64), sc),
                               rtol=1e-13, atol=1e-13)
    # per-block scales act on their own tokens: doubling k_scale of block 1 equals doubling
    # those keys' codes in the exact formula
    ks2 = ks.copy(); ks2[:, :, 1] = 2.0
    k_eff = kc.astype(np.float64); k_eff[:, :, 64:] *= 2.0
    np.testing.assert_allclose(oracle.log_sum_exp_int8(qc, qs, kc, ks2, sc),
                               oracle.log_sum_exp(qc.astype(np.float64), k_eff, sc), rtol=1e-13, atol=1e-13)


def test_attention_rows_equal_full_rows():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 2100, 8))
    k = rng.standard_normal((1, 2, 300, 8))
    v = rng.standard_normal((1, 2, 300, 8))
    rows = np.array([0, 5, 1023, 1024, 2099])
    # equal up to BLAS blocking, which depends on the number of rows in the product
    np.testing.assert_allclose(oracle.attention_rows(q, k, v, rows),
                               oracle.attention(q, k, v)[:, :, rows], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------------------------

def _exact_f32(fr: Fraction) -> float:
    """Round a rational to the nearest float32 (ties to even), by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    fr = abs(fr)
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1
    e = max(e, -126)                       # subnormal range keeps a fixed quantum
    quantum = Fraction(2) ** (e - 23)
    m = fr / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * quantum)


def _round_half_even(fr: Fraction) -> int:
    n = math.floor(fr)
    rem = fr - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def test_quant_golden_worked_examples():
    for case in _load("quant_worked.json")["cases"]:
        x = np.array(case["x"], dtype=np.float32).reshape(1, 1, -1, 1)
        codes, scales = oracle.quantize_blocks(x, x.shape[2])
        assert scales.shape == (1, 1, 1)
        assert float(scales[0, 0, 0]) == case["scale"], case["name"]
        assert codes.ravel().tolist() == case["codes"], case["name"]


def test_quantizer_matches_exact_rational_rounding():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((1, 2, 200, 8)) * rng.choice([1e-3, 1.0, 37.0], (1, 2, 200, 1)))
    x = x.astype(np.float32)
    codes, scales = oracle.quantize_blocks(x, 64)
    for h in range(2):
        for t in range(scales.shape[2]):
            blk = x[0, h, 64 * t:64 * t + 64]
            amax = max(abs(Fraction(float(e))) for e in blk.ravel())
            sc = _exact_f32(amax / 127) if amax else 1.0
            assert float(scales[0, h, t]) == sc
            for i in range(blk.shape[0]):
                for d in range(0, blk.shape[1], 3):
                    qv = _exact_f32(Fraction(float(blk[i, d])) / Fraction(sc))
                    ref = max(-127, min(127, _round_half_even(Fraction(qv))))
                    assert int(codes[0, h, 64 * t + i, d]) == ref


def test_scale_is_a_true_division_for_every_bf16_mantissa():
    # one block per bf16 value in [1, 2): scale must be the correctly rounded amax / 127;
    # multiplying by a rounded reciprocal differs for several of these mantissas
    amax = datagen.bf16_to_f32(np.arange(0x3F80, 0x4000, dtype=np.uint16))
    x = amax.reshape(1, 1, -1, 1)
    _, scales = oracle.quantize_blocks(x, 1)
    for a, s in zip(amax, scales.ravel()):
        assert float(s) == _exact_f32(Fraction(float(a)) / 127)


def test_quantizer_invariants_and_ragged_tail():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2, 3, 300, 16)).astype(np.float32) * 3
    x[1, 2, 256:300] = 0.0                    # tail block of 44 tokens, all zero
    codes, scales = oracle.quantize_blocks(x, 128)
    assert scales.shape == (2, 3, 3)
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    assert scales[1, 2, 2] == np.float32(1.0)
    assert np.all(codes[1, 2, 256:] == 0)
    for b in range(2):
        for h in range(3):
            for t in range(3):
                blk = codes[b, h, 128 * t:128 * t + 128]
                if (b, h, t) != (1, 2, 2):
                    assert np.abs(blk.astype(np.int32)).max() == 127
                err = np.abs(x[b, h, 128 * t:128 * t + 128].astype(np.float64)
                             - blk.astype(np.float64) * float(scales[b, h, t]))
                assert err.max() <= float(scales[b, h, t]) * 0.5 * (1 + 2 ** -20)
    # the tail block's scale sees only its own 44 tokens
    np.testing.assert_equal(scales[0, 0, 2],
                            np.abs(x[0, 0, 256:]).max() / np.float32(127))


def test_k_mean_is_exactly_rounded():
    # adversarial channel: 2^60 + 1 - 2^60 -> naive fp64 summation loses the 1
    k = np.zeros((1, 1, 3, 2))
    k[0, 0, :, 0] = [2.0 ** 60, 1.0, -(2.0 ** 60)]
    k[0, 0, :, 1] = [0.5, 0.25, 0.125]
    m = oracle.k_channel_mean(k)
    assert m[0, 0, 0] == np.float32(1.0 / 3.0)
    assert m[0, 0, 1] == np.float32(0.875 / 3.0)
    rng = np.random.default_rng(12)
    kb = _bf(rng.standard_normal((1, 2, 301, 4)) * 3 + 1.7)
    m = oracle.k_channel_mean(kb)
    for h in range(2):
        for d in range(4):
            exact = sum(Fraction(float(t)) for t in kb[0, h, :, d])
            assert m[0, h, d] == np.float32(float(exact) / 301)


def test_k_mean_shift_and_zero_channel():
    rng = np.random.default_rng(13)
    k = rng.integers(-64, 65, (1, 2, 96, 8)) / 16.0
    c = rng.integers(-3, 4, (1, 2, 1, 8)).astype(np.float64)
    m0 = oracle.k_channel_mean(k).astype(np.float64)
    m1 = oracle.k_channel_mean(k + c).astype(np.float64)
    # exact sums; the means differ by c up to the fp32 rounding of each mean
    np.testing.assert_allclose(m1 - m0, c[:, :, 0, :], rtol=0, atol=2 ** -18)
    k[0, 1, :, 5] = 0.0
    q = oracle.quantize_qk(np.ones((1, 2, 96, 8)), k)
    assert q["k_mean"][0, 1, 5] == 0.0
    assert np.all(q["k_codes"][0, 1, :, 5] == 0)


def test_smoothing_leaves_attention_unchanged():
    rng = np.random.default_rng(14)
    q = _bf(rng.standard_normal((1, 2, 40, 16)))
    k = _bf(rng.standard_normal((1, 2, 70, 16)) + rng.standard_normal((1, 2, 1, 16)) * 4)
    v = _bf(rng.standard_normal((1, 2, 70, 16)))
    mean = oracle.k_channel_mean(k)
    # the exact shift (fp64 holds bf16 minus fp32 exactly) cancels in the softmax
    kx = k - mean.astype(np.float64)[:, :, None, :]
    np.testing.assert_allclose(oracle.attention(q, kx, v), oracle.attention(q, k, v),
                               rtol=1e-12, atol=1e-13)
    # smooth_k is that exact difference rounded once to fp32
    np.testing.assert_array_equal(oracle.smooth_k(k, mean), kx.astype(np.float32))


def test_int8_attention_reduces_to_exact_attention():
    # integer Q, K in [-127, 127]; every block holds +-127 and every K column sums to 0,
    # so the K mean is 0, every scale is 1 and the codes are the values themselves
    rng = np.random.default_rng(15)
    S, D = 256, 16
    q = rng.integers(-126, 127, (1, 2, S, D)).astype(np.float64)
    q[:, :, ::128, 0] = 127
    half = rng.integers(-126, 127, (1, 2, S // 2, D)).astype(np.float64)
    half[:, :, ::32, 1] = 127
    k = np.concatenate([half, -half], axis=2)
    v = _bf(rng.standard_normal((1, 2, S, D)))
    qq = oracle.quantize_qk(q, k)
    assert np.all(qq["k_mean"] == 0) and np.all(qq["q_scale"] == 1) and np.all(qq["k_scale"] == 1)
    np.testing.assert_array_equal(qq["q_codes"], q.astype(np.int8))
    np.testing.assert_array_equal(qq["k_codes"], k.astype(np.int8))
    sc = 1 / 64.0
    got = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v, sc)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, sc), rtol=1e-12, atol=1e-13)


def test_int8_attention_block_scales_map_to_their_tokens():
    # ragged S: Q blocks of 128 (tail 44), K blocks of 64 (tail 44); distinct scales per block
    rng = np.random.default_rng(16)
    S, D = 300, 8
    qc = rng.integers(-127, 128, (1, 1, S, D)).astype(np.int8)
    kc = rng.integers(-127, 128, (1, 1, S, D)).astype(np.int8)
    qs = np.array([[[0.011, 0.02, 0.005]]], dtype=np.float32)
    ks = np.array([[[0.03, 0.001, 0.017, 0.008, 0.025]]], dtype=np.float32)
    v = rng.standard_normal((1, 1, S, D))
    qd = np.empty((S, D)); kd = np.empty((S, D))
    for i in range(S):
        qd[i] = qc[0, 0, i].astype(np.float64) * float(qs[0, 0, i // 128])
        kd[i] = kc[0, 0, i].astype(np.float64) * float(ks[0, 0, i // 64])
    ref = oracle.attention(qd[None, None], kd[None, None], v, 0.3)
    got = oracle.attention_int8(qc, qs, kc, ks, v, 0.3)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    rows = np.array([0, 127, 128, 299])
    np.testing.assert_allclose(oracle.attention_int8(qc, qs, kc, ks, v, 0.3, rows=rows),
                               got[:, :, rows], rtol=1e-13, atol=1e-15)


def test_int8_zero_scale_guard_cases_give_mean_of_v():
    rng = np.random.default_rng(17)
    S, D = 200, 16
    v = _bf(rng.standard_normal((1, 2, S, D)))
    mean_v = v.mean(axis=2, keepdims=True)
    # (i) Q == 0: every Q block has amax 0
    k = _bf(rng.standard_normal((1, 2, S, D)))
    qq = oracle.quantize_qk(np.zeros((1, 2, S, D)), k)
    assert np.all(qq["q_scale"] == 1.0) and np.all(qq["q_codes"] == 0)
    o = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), rtol=0, atol=1e-14)
    # (ii) all K rows identical: smoothed K is exactly 0, every K block has amax 0
    row = _bf(rng.standard_normal(D) * 3)
    kconst = np.broadcast_to(row, (1, 2, S, D)).copy()
    qq = oracle.quantize_qk(_bf(rng.standard_normal((1, 2, S, D))), kconst)
    assert np.all(qq["k_scale"] == 1.0) and np.all(qq["k_codes"] == 0)
    o = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v)
    np.testing.assert_allclose(o, np.broadcast_to(mean_v, o.shape), rtol=0, atol=1e-14)


def test_int8_attention_close_to_exact_on_gaussian_data():
    q, k, v = (datagen.bf16_to_f64(t) for t in datagen.attention_inputs("tiny"))
    qq = oracle.quantize_qk(q, k)
    oq = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v)
    oe = oracle.attention(q, k, v)
    rel = np.linalg.norm(oq - oe) / np.linalg.norm(oe)
    assert 1e-4 < rel < 5e-2


# ---------------------------------------------------------------------------------------------
# relative L1
# ---------------------------------------------------------------------------------------------

def test_rel_l1_golden():
    for case in _load("rel_l1_worked.json")["cases"]:
        r = oracle.rel_l1(np.array(case["a"]), np.array(case["b"]))
        want = float("inf") if case["r"] == "inf" else case["r"]
        assert r == want, case["name"]


def test_rel_l1_brute_force_rational():
    rng = np.random.default_rng(18)
    a = _bf(rng.standard_normal(999))
    b = _bf(rng.standard_normal(999))
    num = sum(abs(Fraction(float(x)) - Fraction(float(y))) for x, y in zip(a, b))
    den = sum(abs(Fraction(float(y))) for y in b)
    assert abs(oracle.rel_l1(a, b) - float(num / den)) <= 1e-15


def test_rel_l1_residual_distribution_statistics():
    a, b = datagen.residual_pair(256, 3072)
    r = oracle.rel_l1(datagen.bf16_to_f64(a), datagen.bf16_to_f64(b))
    # E|0.05 n| / E|b| = 0.05 for independent standard normals n, b
    assert abs(r - 0.05) < 0.05 * 0.01


# ---------------------------------------------------------------------------------------------
# input generator
# ---------------------------------------------------------------------------------------------

def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5],
                 dtype=np.float32)
    got = datagen.bf16_to_f64(datagen.f32_to_bf16_bits(x)).tolist()
    assert got == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5]


def test_generator_deterministic_and_shaped():
    a = datagen.attention_inputs("tiny")
    b = datagen.attention_inputs("tiny")
    for x, y in zip(a, b):
        assert x.shape == (1, 2, 256, 64) and x.dtype == np.uint16
        np.testing.assert_array_equal(x, y)
    qf = datagen.bf16_to_f64(a[0])
    assert abs(qf.mean()) < 0.02 and abs(qf.std() - 1) < 0.02


# ---- quantization-error probe ----------------------------------------------------------------

def test_probe_rows_are_bin_middles():
    for S, R in [(1, 1), (7, 7), (10, 1), (10, 3), (4608, 256), (118800, 256), (129, 64)]:
        rows = oracle.probe_rows(S, R)
        step = S // R
        assert rows.size == R and np.all(np.diff(rows) == step) and rows[-1] < S
        for i, r in enumerate(rows):
            # bin i holds rows [i step, (i + 1) step); r is its middle row (the upper of the two
            # middle rows when step is even)
            lo, hi = i * step, (i + 1) * step
            assert lo <= r < hi and (r - lo) - (hi - 1 - r) in (0, 1)
    assert list(oracle.probe_rows(5, 5)) == [0, 1, 2, 3, 4]
    assert list(oracle.probe_rows(9, 1)) == [4]
    assert list(oracle.probe_rows(10, 3)) == [1, 4, 7]
    assert list(oracle.probe_rows(118800, 256)[:3]) == [232, 696, 1160]


def test_probe_error_zero_when_quantization_is_exact():
    # integer Q, K with +-127 in every block and zero K column sums: codes equal the values
    rng = np.random.default_rng(31)
    S, D = 256, 16
    q = rng.integers(-126, 127, (1, 2, S, D)).astype(np.float64)
    q[:, :, ::128, 0] = 127
    half = rng.integers(-126, 127, (1, 2, S // 2, D)).astype(np.float64)
    half[:, :, ::32, 1] = 127
    k = np.concatenate([half, -half], axis=2)
    v = _bf(rng.standard_normal((1, 2, S, D)))
    overall, per_head = oracle.quant_probe_error(q, k, v, 32, scale=1 / 64.0)
    assert overall <= 1e-12 and np.all(per_head <= 1e-12)


def test_probe_error_brute_force_aggregation():
    rng = np.random.default_rng(32)
    B, H, S, D, R = 2, 2, 150, 16, 7
    q, k, v = (_bf(rng.standard_normal((B, H, S, D))) for _ in range(3))
    overall, per_head = oracle.quant_probe_error(q, k, v, R)
    full_exact = oracle.attention(q, k, v)
    qq = oracle.quantize_qk(q, k)
    full_quant = oracle.attention_int8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v)
    tot_num = tot_den = 0.0
    for b in range(B):
        for h in range(H):
            num = den = 0.0
            for i in range(R):
                row = (S // R) // 2 + i * (S // R)
                for d in range(D):
                    num += (full_quant[b, h, row, d] - full_exact[b, h, row, d]) ** 2
                    den += full_exact[b, h, row, d] ** 2
            assert abs(per_head[b, h] - math.sqrt(num / den)) <= 1e-12
            tot_num += num
            tot_den += den
    assert abs(overall - math.sqrt(tot_num / tot_den)) <= 1e-12
    assert 1e-3 < overall < 0.1   # int8 error of Gaussian inputs: small but not zero
