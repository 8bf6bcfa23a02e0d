"""Pins of the oracle's estimator factors (CPU): a planted spectrum is
recovered, full rank reproduces the weight, the truncation error is the tail of
the spectrum (Eckart-Young, with the spectrum from a different routine), and
the sign rule holds."""
import numpy as np

from oracle import reference as ref


def _orth(rng, n, m):
    q, _ = np.linalg.qr(rng.standard_normal((n, m)))
    return q


def test_planted_spectrum_recovered(rng):
    d_in, d_out, n, k = 40, 70, 30, 6
    U0, V0 = _orth(rng, d_in, n), _orth(rng, d_out, n)
    s0 = 5.0 * 0.8 ** np.arange(n)
    W_lin = (U0 * s0 @ V0.T).T                       # W = U0 S V0^T, W_lin = W^T
    WA_t, WB = ref.svd_factors(W_lin, k)
    for j in range(k):
        u = U0[:, j] * np.sign(U0[np.argmax(np.abs(U0[:, j])), j])
        v = V0[:, j] * np.sign(U0[np.argmax(np.abs(U0[:, j])), j])
        assert np.allclose(WA_t[j], np.sqrt(s0[j]) * u, atol=1e-12)
        assert np.allclose(WB[j], np.sqrt(s0[j]) * v, atol=1e-12)


def test_full_rank_reproduces_weight_and_tail_error(rng):
    W_lin = rng.standard_normal((25, 18))
    WA_t, WB = ref.svd_factors(W_lin, 18)
    assert np.allclose(WA_t.T @ WB, W_lin.T, atol=1e-12)
    lam = np.sort(np.linalg.eigvalsh(W_lin @ W_lin.T))[::-1]     # squared singular values
    for k in (1, 5, 12):
        WA_t, WB = ref.svd_factors(W_lin, k)
        err = np.sum((W_lin.T - WA_t.T @ WB) ** 2)
        assert np.isclose(err, np.sum(np.maximum(lam[k:18], 0.0)), rtol=1e-10, atol=1e-10)


def test_sign_rule(rng):
    WA_t, _ = ref.svd_factors(rng.standard_normal((30, 20)), 7)
    for row in WA_t:
        assert row[np.argmax(np.abs(row))] > 0
