"""Pins of the oracle's criterion ablations (CPU): exact-output ("oracle")
criterion, random selection, head-level QK selection.

Pages: "SparseLoRA: Accelerating LLM Fine-Tuning with Contextual Sparsity",
paper-graph summary §3.4 "Oracle Sparse Neuron Selection Criteria" (Table 7's
oracle row), "Why not head-level pruning for QK?", and the pruning-criterion
ablation (Table 10: random, head-level).  The random generator is SplitMix64
(Steele, Lea and Flood, 2014)."""
import numpy as np
import pytest

from oracle import csa


def test_random_scores_published_splitmix64_outputs():
    """From state 0 SplitMix64's first three outputs are 0xe220a8397b1dcdaf,
    0x6e789e6aa1b965f4, 0x06c45d188009454f (the generator's reference
    implementation); the scores are their top 24 bits over 2^24."""
    want = np.array([(v >> 40) / 2.0 ** 24 for v in
                     (0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F)], np.float32)
    assert np.array_equal(csa.random_scores(0, 3), want)


def test_random_scores_range_grid_and_uniformity():
    s = csa.random_scores(123456789, 1 << 20)
    assert s.dtype == np.float32 and s.min() >= 0.0 and s.max() < 1.0
    assert np.array_equal(s * np.float32(2 ** 24), np.floor(s.astype(np.float64) * 2 ** 24))
    # mean 1/2 and variance 1/12 within 6 standard errors of a uniform sample
    n = s.size
    assert abs(s.mean() - 0.5) < 6 * np.sqrt(1 / 12 / n)
    assert abs(s.var() - 1 / 12) < 6 * np.sqrt(1 / 180 / n)
    # different seeds give different draws; a seed shifted by the generator's
    # increment is the same sequence one counter later
    assert not np.array_equal(s[:64], csa.random_scores(123456790, 64))
    gamma = 0x9E3779B97F4A7C15
    assert np.array_equal(csa.random_scores(123456789 + gamma, 63), s[1:64])


def test_random_selection_is_uniform_over_channels():
    """Kept-channel frequencies over many seeds are flat (each channel kept with
    probability n/C)."""
    C, n, trials = 40, 10, 4000
    cnt = np.zeros(C)
    for t in range(trials):
        cnt[csa.select(csa.random_scores(t * 7919, C), n)] += 1
    p = n / C
    sd = np.sqrt(trials * p * (1 - p))
    assert np.all(np.abs(cnt - trials * p) < 5 * sd)


def test_dense_l2_integer_data_is_exact(rng):
    Y = rng.integers(-8, 9, size=(300, 37)).astype(np.float32)
    rows = np.sort(rng.choice(300, 211, replace=False))
    got = csa.dense_ssq("l2", Y, None, rows)
    want = (Y[rows].astype(np.int64) ** 2).sum(0)
    assert np.array_equal(got, want.astype(np.float32))


def test_dense_swiglu_near_fp64(rng):
    G = rng.standard_normal((200, 29)).astype(np.float32) * 3
    U = rng.standard_normal((200, 29)).astype(np.float32)
    rows = np.arange(0, 200, 3)
    g, u = G[rows].astype(np.float64), U[rows].astype(np.float64)
    want = ((g / (1 + np.exp(-g)) * u) ** 2).sum(0)
    assert np.max(np.abs(csa.dense_ssq("swiglu", G, U, rows) - want) / want) < 1e-5


def test_dense_criterion_is_the_estimator_with_identity_factors(rng):
    """With xa = the exact outputs of the listed rows and W_B = I, the
    estimator's second stage returns those outputs exactly, so its criteria
    (pinned on their own) equal the exact-output criteria bit for bit."""
    T, C = 90, 24
    G = rng.standard_normal((T, C)).astype(np.float32)
    U = rng.standard_normal((T, C)).astype(np.float32)
    rows = np.sort(rng.choice(T, 70, replace=False))
    eye = np.eye(C, dtype=np.float32)
    xa = np.ascontiguousarray(np.concatenate([G[rows], U[rows]], 1))
    assert np.array_equal(csa.dense_ssq("l2", G, None, rows), csa.ssq_l2(xa, eye, off=0))
    assert np.array_equal(csa.dense_ssq("swiglu", G, U, rows), csa.ssq_swiglu(xa, eye, eye, 0, C))


def test_dense_qk_grouping(rng):
    """QK on exact outputs: a query channel (g n_rep + r) d + j feeds key/value
    channel g d + j; MHA reduces to the plain product of the two L2 sums."""
    H, n_rep, d, T = 3, 2, 4, 10
    rows = np.arange(T)
    K = rng.standard_normal((T, H * d)).astype(np.float32)
    for g in range(H):
        for r in range(n_rep):
            for j in range(d):
                Q = np.zeros((T, H * n_rep * d), np.float32)
                Q[:, (g * n_rep + r) * d + j] = 1.0
                s = csa.dense_scores("qk", Q, K, rows, H, n_rep, d)
                nz = np.flatnonzero(s)
                assert list(nz) == [g * d + j]
    Q = rng.standard_normal((T, H * d)).astype(np.float32)
    s = csa.dense_scores("qk", Q, K, rows, H, 1, d)
    assert np.array_equal(s, (csa.dense_ssq("l2", Q, None, rows) * csa.dense_ssq("l2", K, None, rows)))


def test_head_scores_and_selection_hand_case():
    s = np.array([1, 2, 3, 4, 5, 6, 0.5, 0.5, 0.5], np.float32)
    assert np.array_equal(csa.head_scores(s, 3, 3), np.array([6, 15, 1.5], np.float32))
    assert list(csa.select_heads(s, 3, 3, 1)) == [3, 4, 5]
    assert list(csa.select_heads(s, 3, 3, 2)) == [0, 1, 2, 3, 4, 5]
    # equal head scores: the lower head index is kept
    t = np.array([1, 1, 2, 0, 0, 2], np.float32)
    assert list(csa.select_heads(t, 3, 2, 1)) == [0, 1]


def test_head_selection_brute_force(rng):
    for _ in range(30):
        H, d = int(rng.integers(1, 9)), int(rng.integers(1, 6))
        s = rng.integers(0, 4, size=H * d).astype(np.float32)    # many ties
        h = int(rng.integers(0, H + 1))
        hs = [float(np.float32(sum(np.float32(v) for v in s[g * d:(g + 1) * d]))) for g in range(H)]
        keep = sorted(sorted(range(H), key=lambda g: (-hs[g], g))[:h])
        want = [g * d + j for g in keep for j in range(d)]
        assert list(csa.select_heads(s, H, d, h)) == want
