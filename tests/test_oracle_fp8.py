"""Pins of the fp8 (OCP e4m3) part of the oracle: code values and rounding against torch's
float8_e4m3fn and against exact rational rounding, the block quantizer's contract, and the
reduction of fp8 attention to exact attention when the codes are the values."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _grid():
    """All non-negative finite e4m3 values, by the definition of the format."""
    vals = [Fraction(m, 8) * Fraction(1, 64) for m in range(8)]            # subnormals
    for e in range(1, 16):
        for m in range(8):
            if e == 15 and m == 7:
                continue                                                   # NaN
            vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


def _exact_round(fr: Fraction) -> float:
    """Nearest e4m3 value to a rational of magnitude <= 448, ties to the even fraction field."""
    g = _grid()
    a = abs(fr)
    best = min(range(len(g)), key=lambda i: (abs(g[i] - a), i % 2))   # index parity = m parity
    v = float(g[best])
    return -v if fr < 0 else v


def test_code_values_match_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(codes)
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.e4m3_value(np.array([0x7E]))[0] == oracle.E4M3_MAX == 448.0
    assert [float(x) for x in _grid()] == list(oracle.e4m3_value(np.arange(127, dtype=np.uint8)))


def test_rounding_matches_exact_rational_rounding():
    g = _grid()
    mids = [(g[i] + g[i + 1]) / 2 for i in range(len(g) - 1)]
    xs = mids + [m + Fraction(1, 1 << 20) for m in mids] + [m - Fraction(1, 1 << 20) for m in mids]
    rng = np.random.default_rng(40)
    xs += [Fraction(float(v)) for v in rng.uniform(-448, 448, 300)]
    xs += [Fraction(float(v)) for v in rng.standard_normal(200) * 2.0 ** rng.integers(-12, 4, 200)]
    xs += [Fraction(0), Fraction(448), Fraction(-448), Fraction(1, 1 << 12)]
    vals = np.array([float(x) for x in xs])
    got = oracle.e4m3_value(oracle.e4m3_round(vals))
    for x, gv in zip(xs, got):
        assert gv == _exact_round(x), (float(x), gv)


def test_rounding_matches_torch_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(41)
    x = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 6, 20000)])
    x = np.clip(x, -448, 448).astype(np.float32)
    g = np.array([float(v) for v in _grid()])
    x = np.concatenate([x, ((g[1:] + g[:-1]) / 2).astype(np.float32)])   # every tie
    x = np.concatenate([x, np.array([-1e-5, 1e-5, -0.0, 0.0, -0.00097, -0.00098], np.float32)])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_round(x.astype(np.float64))
    assert np.array_equal(got, ref), x[got != ref][:5]


def test_rounding_keeps_the_sign_of_zero_results():
    # half the smallest subnormal (2^-10) and below round to zero, keeping the sign
    assert list(oracle.e4m3_round(np.array([2.0 ** -11, -2.0 ** -11, -0.0, 0.0, -2.0 ** -10,
                                            -2.0 ** -10 * 1.01]))) == [0x00, 0x80, 0x80, 0x00,
                                                                       0x80, 0x81]


def test_block_quantizer_contract():
    rng = np.random.default_rng(42)
    B, H, S, D = 1, 2, 300, 64
    x = (rng.standard_normal((B, H, S, D)) * 3).astype(np.float32)
    x[0, 1, 64:128] = 0                                     # an all-zero K block
    codes, scales = oracle.quantize_blocks_fp8(x, 64)
    assert scales.shape == (B, H, 5) and scales[0, 1, 1] == 1.0 and not codes[0, 1, 64:128].any()
    vals = oracle.e4m3_value(codes)
    for h in range(H):
        for t in range(5):
            blk = x[0, h, 64 * t:min(S, 64 * (t + 1))]
            sc = scales[0, h, t]
            if not blk.any():
                continue
            amax = np.abs(blk).max()
            assert sc == np.float32(amax) / np.float32(448)
            # the element holding amax maps to +-448 exactly
            i = np.unravel_index(np.abs(blk).argmax(), blk.shape)
            assert abs(vals[0, h, 64 * t + i[0], i[1]]) == 448.0
            # one rounding: within half a step of the quotient (relative 2^-4 for normal
            # values, 2^-10 absolute below 2^-6)
            qv = (blk / sc).astype(np.float64)
            dec = vals[0, h, 64 * t:64 * t + blk.shape[0]]
            bound = np.maximum(np.abs(qv) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-12)
            assert np.all(np.abs(dec - qv) <= bound)


def test_fp8_attention_reduces_to_exact_attention():
    # Q, K on the e4m3 grid with 448 in every block and zero K column sums: the K mean is 0,
    # every scale is 1 and the codes are the values, so the fp8 attention is exact attention
    rng = np.random.default_rng(43)
    S, D = 256, 16
    g = oracle.e4m3_value(np.arange(127, dtype=np.uint8))
    def grid_values(shape):
        return rng.choice(g[40:110], size=shape) * rng.choice([-1.0, 1.0], size=shape)
    q = grid_values((1, 2, S, D))
    q[:, :, ::128, 0] = 448.0
    half = grid_values((1, 2, S // 2, D))
    half[:, :, ::32, 1] = 448.0
    k = np.concatenate([half, -half], axis=2)
    v = rng.standard_normal((1, 2, S, D))
    qq = oracle.quantize_qk_fp8(q, k)
    assert np.all(qq["k_mean"] == 0) and np.all(qq["q_scale"] == 1) and np.all(qq["k_scale"] == 1)
    assert np.array_equal(oracle.e4m3_value(qq["q_codes"]), q)
    assert np.array_equal(oracle.e4m3_value(qq["k_codes"]), k)
    sc = 1 / 2048.0
    got = oracle.attention_fp8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], v, sc)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, sc), rtol=1e-12, atol=1e-13)
    lse = oracle.log_sum_exp_fp8(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"], sc)
    np.testing.assert_allclose(lse, oracle.log_sum_exp(q, k, sc), rtol=1e-12, atol=1e-12)


def test_v_quantizer_per_channel_contract():
    rng = np.random.default_rng(44)
    v = rng.standard_normal((2, 3, 200, 16)) * np.linspace(0.1, 10, 16)
    v[1, 2, :, 5] = 0.0                                     # an all-zero channel
    codes, scales = oracle.quantize_v_fp8(v)
    assert codes.shape == v.shape and scales.shape == (2, 3, 16)
    assert scales[1, 2, 5] == 1.0 and not codes[1, 2, :, 5].any()
    vals = oracle.e4m3_value(codes)
    vf = v.astype(np.float32)
    for b in range(2):
        for h in range(3):
            for d in range(16):
                col = vf[b, h, :, d]
                if not col.any():
                    continue
                amax = np.abs(col).max()
                assert scales[b, h, d] == np.float32(amax) / np.float32(448)
                assert np.abs(vals[b, h, :, d]).max() == 448.0          # the amax token
                qv = (col / scales[b, h, d]).astype(np.float64)
                bound = np.maximum(np.abs(qv) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-12)
                assert np.all(np.abs(vals[b, h, :, d] - qv) <= bound)


def test_full_fp8_attention_reduces_to_exact_attention():
    # V on the e4m3 grid with 448 in every channel: scale 1, codes = values; with exact Q/K
    # codes too (construction of the QK test above), the result is exact attention
    rng = np.random.default_rng(45)
    S, D = 256, 16
    g = oracle.e4m3_value(np.arange(127, dtype=np.uint8))
    def grid_values(shape):
        return rng.choice(g[40:110], size=shape) * rng.choice([-1.0, 1.0], size=shape)
    q = grid_values((1, 2, S, D))
    q[:, :, ::128, 0] = 448.0
    half = grid_values((1, 2, S // 2, D))
    half[:, :, ::32, 1] = 448.0
    k = np.concatenate([half, -half], axis=2)
    v = grid_values((1, 2, S, D))
    v[:, :, 7, :] = 448.0
    qq = oracle.quantize_qk_fp8(q, k)
    vc, vs = oracle.quantize_v_fp8(v)
    assert np.all(vs == 1.0) and np.array_equal(oracle.e4m3_value(vc), v)
    sc = 1 / 2048.0
    got = oracle.attention_fp8_full(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"],
                                    vc, vs, sc)
    np.testing.assert_allclose(got, oracle.attention(q, k, v, sc), rtol=1e-12, atol=1e-9)
    # and V scales that are not 1 are applied per channel: a power of two per channel keeps the
    # codes and scales exact, and each output channel scales by its own factor
    f = 2.0 ** (np.arange(D) % 7 - 3.0)
    vc2, vs2 = oracle.quantize_v_fp8(v * f)
    assert np.array_equal(vs2[0, 0], f.astype(np.float32)) and np.array_equal(vc2, vc)
    got2 = oracle.attention_fp8_full(qq["q_codes"], qq["q_scale"], qq["k_codes"], qq["k_scale"],
                                     vc2, vs2, sc)
    np.testing.assert_allclose(got2, got * f, rtol=1e-12, atol=1e-9)


def test_fp8_k_smoothing_invariance():
    # a per-channel constant added to K moves the K mean by that constant and leaves the
    # smoothed K, hence its codes and scales, unchanged (S a power of two and dyadic values, so
    # the mean and every difference are exact in fp32)
    rng = np.random.default_rng(46)
    S, D = 256, 16
    k = np.round(rng.standard_normal((1, 2, S, D)) * 64) / 64
    q = np.round(rng.standard_normal((1, 2, S, D)) * 64) / 64
    c = np.round(rng.standard_normal((1, 2, 1, D)) * 8) * 4          # multiples of 4, up to ~100
    a = oracle.quantize_qk_fp8(q, k)
    b = oracle.quantize_qk_fp8(q, k + c)
    np.testing.assert_array_equal(b["k_mean"], (a["k_mean"] + c[:, :, 0].astype(np.float32)))
    assert np.array_equal(b["k_codes"], a["k_codes"]) and np.array_equal(b["k_scale"], a["k_scale"])
    assert np.array_equal(b["q_codes"], a["q_codes"])
