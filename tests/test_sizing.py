"""Pins for the predictor sizing study (CPU only)."""
import numpy as np
import pytest

from activation_sparse_predict_amd import sizing


def test_spectral_matrix_has_the_requested_spectrum():
    rng = np.random.default_rng(1)
    f, d, alpha = 96, 32, 0.7
    W = sizing.spectral_matrix(rng, f, d, alpha)
    s = np.linalg.svd(W, compute_uv=False)
    want = np.arange(1, d + 1, dtype=np.float64) ** -alpha
    want *= np.sqrt(f / np.sum(want ** 2))
    np.testing.assert_allclose(s, want, rtol=1e-10)
    assert np.mean(np.sum(W * W, axis=1)) == pytest.approx(1.0, rel=1e-10)   # mean squared row norm 1


def test_rank_r_predictor_is_the_best_rank_r_approximation():
    """Eckart-Young: |W - B A|_F^2 is the sum of the squared singular values past r."""
    rng = np.random.default_rng(2)
    W = rng.standard_normal((40, 24))
    s = np.linalg.svd(W, compute_uv=False)
    for r in (1, 5, 24):
        A, B = sizing.rank_r_predictor(W, r)
        assert A.shape == (r, 24) and B.shape == (40, r)
        assert np.sum((W - B @ A) ** 2) == pytest.approx(np.sum(s[r:] ** 2), rel=1e-9, abs=1e-9)


def test_full_rank_predicts_exactly_and_rank_zero_is_the_bias():
    rng = np.random.default_rng(3)
    f, d = 64, 16
    W = rng.standard_normal((f, d))
    bias = rng.standard_normal(f)
    X = rng.standard_normal((50, d))
    A, B = sizing.rank_r_predictor(W, d)
    q = sizing.predictor_quality(W, bias, A, B, X)
    assert q["recall"] == 1.0 and q["precision"] == 1.0
    A0, B0 = np.zeros((0, d)), np.zeros((f, 0))
    q0 = sizing.predictor_quality(W, bias, A0, B0, X)
    truth = X @ W.T + bias > 0
    pred = np.broadcast_to(bias > 0, truth.shape)
    assert q0["recall"] == pytest.approx(np.sum(truth & pred) / np.sum(truth))
    assert q0["predicted_rate"] == pytest.approx(np.mean(bias > 0))


def test_study_rates_and_monotone_recall():
    rows = sizing.study(d=128, f=512, ranks=(4, 16, 64, 128), alphas=(1.0,), tokens=64, seed=5)
    rec = [q["recall"] for q in rows]
    assert all(b >= a - 1e-12 for a, b in zip(rec, rec[1:]))
    assert rows[-1]["recall"] == 1.0 and rows[-1]["precision"] == 1.0   # full rank
    assert 0.05 < rows[0]["true_rate"] < 0.15                          # Zipf rates of mean 0.1
    assert rows[0]["byte_ratio"] == pytest.approx((4 * 128 + 512 * 4) / (512 * 128))
