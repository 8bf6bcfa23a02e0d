"""Pins of the oracle's fp32 score path against what mathematics fixes.

Nothing here retypes the oracle: each check is a closed form, an exact
result, an error bound around an fp64 / exact-rational value, or a special
case that reduces to a library routine.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import csa, reference as ref
from tests.fp32exact import gamma, ln2_fraction, r64_bound, round_f32
from workloads.gen import round_dtype, svd_factor_pair


# ---------------------------------------------------------------- exp / SiLU

def test_exp_constants_are_correctly_rounded():
    ln2 = ln2_fraction()
    c = csa.exp_constants()
    assert c[0] == round_f32(1 / ln2)                      # LOG2E
    hi = Fraction(round(ln2 * 4096), 4096)                 # 12 significant bits
    assert Fraction(float(c[1])) == hi
    assert c[2] == round_f32(ln2 - hi)                     # LN2_LO
    for i in range(8):
        assert c[3 + i] == round_f32(Fraction(1, math.factorial(i)))
    # n * LN2_HI exact for |n| <= 150: LN2_HI has at most 12 significant bits
    m = Fraction(float(c[1])) * 4096
    assert m.denominator == 1 and int(m).bit_length() <= 12


def test_exp_sl_within_two_ulp_on_strided_sweep():
    worst, cnt = csa.exp_sweep(stride=61, lo=-104.0, hi=89.0)
    assert cnt > 10_000_000
    assert worst <= 1.0, worst          # the exhaustive sweep gives 0.939 ulp


def test_exp_sl_special_values():
    z = np.array([0.0, -0.0, 1.0, np.nan, 89.0, 1e30, np.inf, -104.0, -1e30, -np.inf,
                  88.5, -103.5, 88.72283], np.float32)
    e = csa.exp_sl(z)
    assert e[0] == 1.0 and e[1] == 1.0
    assert abs(float(e[2]) - math.e) <= 2 * 2.0 ** -23 * math.e
    assert np.isnan(e[3])
    assert np.isposinf(e[4]) and np.isposinf(e[5]) and np.isposinf(e[6])
    assert e[7] == 0.0 and e[8] == 0.0 and e[9] == 0.0
    assert np.isfinite(e[10]) and e[10] > 1e38
    assert 0.0 < e[11] < 1.2e-38                            # gradual underflow
    assert np.isfinite(e[12]) or e[12] == np.inf


def test_silu_sl_near_fp64(rng):
    z = np.concatenate([rng.uniform(-30, 30, 200_000), rng.uniform(-100, 100, 50_000)])
    z = z.astype(np.float32)
    got = csa.silu_sl(z).astype(np.float64)
    exact = ref.silu(z.astype(np.float64))
    tol = 4 * 2.0 ** -24 * np.abs(exact) + 2.0 ** -149
    ok = z > -88.7                      # below, exp_sl(-z) overflows to +inf by design
    assert np.all(np.abs(got - exact)[ok] <= tol[ok])
    assert np.all(np.abs(got - exact)[~ok] <= 1e-36)
    # silu(0) = 0, silu is odd-symmetric up to the sigmoid: silu(z) - silu(-z) = z
    assert csa.silu_sl(np.float32([0.0]))[0] == 0.0


# ---------------------------------------------------------------- R64

def test_r64_integer_inputs_are_exact(rng):
    for L in (0, 1, 5, 63, 64, 65, 127, 1000, 4097):
        a = rng.integers(-8, 9, L).astype(np.float32)
        b = rng.integers(-8, 9, L).astype(np.float32)
        assert csa.r64(a, b) == np.float32(int(np.dot(a.astype(np.int64), b.astype(np.int64))))


def test_r64_single_nonzero_term_and_position(rng):
    # every position m must contribute exactly once
    L = 300
    for m in (0, 1, 63, 64, 65, 255, 299):
        a = np.zeros(L, np.float32)
        b = np.ones(L, np.float32)
        a[m] = np.float32(1.75)
        assert csa.r64(a, b) == np.float32(1.75)


def test_r64_error_bound(rng):
    for L in (10, 64, 777, 4096, 14336):
        a = rng.standard_normal(L).astype(np.float32)
        b = rng.standard_normal(L).astype(np.float32)
        exact = float(sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, b)))
        bound = r64_bound(L) * float(np.sum(np.abs(a.astype(np.float64) * b)))
        assert abs(float(csa.r64(a, b)) - exact) <= bound


# ---------------------------------------------------------------- stage 1

def test_stage1_rows_and_bound(rng):
    T, D, kt = 50, 300, 7
    x = round_dtype(rng.standard_normal((T, D)), "bf16")
    WA_t = rng.standard_normal((kt, D)).astype(np.float32)
    rows = np.array([3, 0, 17, 49, 22, 5], np.int32)           # any order
    xa = csa.stage1(x, rows, WA_t)
    exact = x[rows].astype(np.float64) @ WA_t.T.astype(np.float64)
    mag = np.abs(x[rows].astype(np.float64)) @ np.abs(WA_t.T.astype(np.float64))
    assert np.all(np.abs(xa - exact) <= r64_bound(D) * mag + 1e-300)
    assert csa.stage1(x, np.zeros(0, np.int32), WA_t).shape == (0, kt)


def test_stage1_identity_factor_returns_x_exactly(rng):
    T, D = 20, 130
    x = round_dtype(rng.standard_normal((T, D)), "bf16")
    rows = np.arange(0, T, 2, dtype=np.int32)
    xa = csa.stage1(x, rows, np.eye(D, dtype=np.float32))
    assert np.array_equal(xa.view(np.uint32), x[rows].view(np.uint32))


# ---------------------------------------------------------------- criteria

def _margin_ok(scores64, n, rel):
    s = np.sort(scores64)[::-1]
    if n == 0 or n == s.size:
        return True
    return (s[n - 1] - s[n]) > rel * s[n - 1] * 4


def _top_set(scores64, n):
    order = np.lexsort((np.arange(scores64.size), -scores64))
    return np.sort(order[:n])


def test_l2_closed_form(rng):
    Tc, k, C = 200, 6, 90
    xa = rng.standard_normal((Tc, k)).astype(np.float32)
    WB = rng.standard_normal((k, C)).astype(np.float32)
    got = csa.ssq_l2(xa, WB).astype(np.float64)
    G = xa.T.astype(np.float64) @ xa.astype(np.float64)
    closed = np.einsum("jc,jl,lc->c", WB.astype(np.float64), G, WB.astype(np.float64))
    # each y_hat carries k fma roundings, the square one, the sum R64(Tc)
    rel = gamma(k) * 2 + r64_bound(Tc) + gamma(2)
    yabs = np.abs(xa.astype(np.float64)) @ np.abs(WB.astype(np.float64))
    bound = rel * np.sum(yabs ** 2, axis=0) * 1.01
    assert np.all(np.abs(got - closed) <= bound)
    # the offset argument selects the right xa columns
    xa2 = np.concatenate([rng.standard_normal((Tc, 3)).astype(np.float32), xa], axis=1)
    assert np.array_equal(csa.ssq_l2(xa2, WB, off=3), csa.ssq_l2(xa, WB))


def test_swiglu_criterion_fp64(rng):
    Tc, k, C = 150, 5, 70
    xa = rng.standard_normal((Tc, 2 * k)).astype(np.float32)
    WBg = rng.standard_normal((k, C)).astype(np.float32)
    WBu = rng.standard_normal((k, C)).astype(np.float32)
    got = csa.ssq_swiglu(xa, WBg, WBu).astype(np.float64)
    g = xa[:, :k].astype(np.float64) @ WBg.astype(np.float64)
    u = xa[:, k:].astype(np.float64) @ WBu.astype(np.float64)
    h = ref.silu(g) * u
    exact = np.sum(h * h, axis=0)
    assert np.all(np.abs(got - exact) <= 2e-5 * np.sum(np.abs(h) ** 2, axis=0) + 1e-30)
    # swapping gate and up changes the result (the gate goes through SiLU)
    assert not np.array_equal(got, csa.ssq_swiglu(xa[:, ::-1].copy(), WBu, WBg))


def test_qk_combine_mha_is_plain_product(rng):
    Q = rng.random(256).astype(np.float32)
    K = rng.random(256).astype(np.float32)
    assert np.array_equal(csa.qk_combine(Q, K, 2, 1, 128), Q * K)


def test_qk_combine_group_mapping(rng):
    H_kv, n_rep, d = 3, 4, 8
    for h in range(H_kv * n_rep):
        for j in (0, 5):
            Q = np.zeros(H_kv * n_rep * d, np.float32)
            Q[h * d + j] = 2.0
            s = csa.qk_combine(Q, np.ones(H_kv * d, np.float32), H_kv, n_rep, d)
            nz = np.nonzero(s)[0]
            assert list(nz) == [(h // n_rep) * d + j]
    Q = rng.random(H_kv * n_rep * d).astype(np.float32)
    K = rng.random(H_kv * d).astype(np.float32)
    exact = Q.astype(np.float64).reshape(H_kv, n_rep, d).sum(1).reshape(-1) * K
    assert np.allclose(csa.qk_combine(Q, K, H_kv, n_rep, d), exact, rtol=gamma(n_rep + 1), atol=0)


def test_identity_factors_reproduce_dense_criterion(rng):
    """With W_A = I and W_B = W (an exact factorisation) the estimator's scores
    are the oracle criterion of the dense output, and the selection equals the
    one from fp64 dense scores whenever the cut has a margin."""
    T, D, C = 96, 64, 120
    roles = (np.arange(T) % 32 >= 24).astype(np.uint8)
    ctx, _ = ref.token_lists(roles)
    x = round_dtype(rng.standard_normal((T, D)), "bf16")
    W = round_dtype(rng.standard_normal((C, D)) * 0.1, "bf16")    # nn.Linear layout
    xa = csa.stage1(x, ctx, np.eye(D, dtype=np.float32))
    sc = csa.ssq_l2(xa, np.ascontiguousarray(W.T))
    y = x[ctx].astype(np.float64) @ W.T.astype(np.float64)
    s64 = np.sum(y * y, axis=0)
    assert np.allclose(sc, s64, rtol=3 * (gamma(D) + r64_bound(len(ctx))), atol=0)
    n = ref.n_keep(C, 7, 10)
    assert _margin_ok(s64, n, 1e-5)
    assert np.array_equal(csa.select(sc, n), _top_set(s64, n))
    # FFN criterion with identity factors for gate and up
    Wu = round_dtype(rng.standard_normal((C, D)) * 0.1, "bf16")
    xa2 = csa.stage1(x, ctx, np.concatenate([np.eye(D), np.eye(D)]).astype(np.float32))
    sc2 = csa.ssq_swiglu(xa2, np.ascontiguousarray(W.T), np.ascontiguousarray(Wu.T))
    h = ref.silu(y) * (x[ctx].astype(np.float64) @ Wu.T.astype(np.float64))
    s2 = np.sum(h * h, axis=0)
    assert np.allclose(sc2, s2, rtol=1e-4, atol=0)
    n = ref.n_keep(C, 1, 2)
    assert _margin_ok(s2, n, 1e-4)
    assert np.array_equal(csa.select(sc2, n), _top_set(s2, n))


def test_full_rank_svd_estimator_matches_dense_selection(rng):
    T, D, C = 80, 48, 100
    roles = (np.arange(T) % 40 >= 30).astype(np.uint8)
    ctx, _ = ref.token_lists(roles)
    x = round_dtype(rng.standard_normal((T, D)), "bf16")
    Wg = round_dtype(rng.standard_normal((C, D)) * 0.1, "bf16")
    Wu = round_dtype(rng.standard_normal((C, D)) * 0.1, "bf16")
    WAg, WBg = svd_factor_pair(Wg, D)
    WAu, WBu = svd_factor_pair(Wu, D)
    xa = csa.stage1(x, ctx, np.concatenate([WAg, WAu]))
    sc = csa.ssq_swiglu(xa, WBg, WBu)
    xc = x[ctx].astype(np.float64)
    h = ref.silu(xc @ Wg.T.astype(np.float64)) * (xc @ Wu.T.astype(np.float64))
    s64 = np.sum(h * h, axis=0)
    assert np.allclose(sc, s64, rtol=1e-3, atol=0)
    for num, den in ((1, 2), (7, 10), (0, 1), (1, 1)):
        n = ref.n_keep(C, num, den)
        if _margin_ok(s64, n, 1e-3):
            assert np.array_equal(csa.select(sc, n), _top_set(s64, n))


def test_scores_are_nonnegative(rng):
    xa = rng.standard_normal((100, 8)).astype(np.float32)
    WB = rng.standard_normal((4, 50)).astype(np.float32)
    for s in (csa.ssq_l2(xa, WB), csa.ssq_swiglu(xa, WB, WB)):
        assert np.all(s.view(np.uint32) < 0x80000000)


def _r64_golden():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "r64_order.json")
    with open(path) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _r64_golden(), ids=lambda c: c["name"][:30])
def test_r64_rounding_order_golden(case):
    """Hand-derived binary32 results that depend on the reduction's order, the
    fused multiply-add and the tree's pairing: the oracle's R64 gives exactly
    the canonical value, which differs from the other orders' values."""
    L = case["L"]
    a = np.zeros(L, np.float32)
    b = np.zeros(L, np.float32)
    for m, av, bv in case["terms"]:
        a[m], b[m] = av, bv
    got = csa.r64(a, b)
    assert np.float32(got).view(np.uint32) == np.float32(case["r64"]).view(np.uint32)
    others = [v for k, v in case.items() if k not in ("name", "terms", "L", "derivation", "r64")]
    assert others and all(np.float32(v) != np.float32(case["r64"]) for v in others)
