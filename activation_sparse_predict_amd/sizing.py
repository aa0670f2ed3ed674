"""Predictor sizing study (CPU, NumPy): how well a rank-r predictor reproduces
the FFN's true activations, and what it costs in bytes.

The pages size the predictor per layer: a smaller predictor for a layer whose
activations are easier to predict, a larger one otherwise, trading accuracy
against the predictor's own memory and time (unite.ai article, "Adaptive
Sparsity-Prädiktoren"; GeekNews summary, adaptive predictor).  Real predictors
are trained; here a *correlated* predictor is built without training: the
rank-r truncated SVD of the up (or gate) matrix W = U diag(sigma) V^T gives
B = U_r and A = diag(sigma_r) V_r^T, so that B (A x) is the best rank-r
approximation of W x, and s = B A x + b uses the neuron's own bias.  How good
that is depends on W's singular spectrum, so the study draws W with a chosen
spectrum sigma_k ~ k^(-alpha) (alpha = 0: the flat spectrum of an i.i.d.
Gaussian matrix) and measures, over tokens x ~ N(0, I):

  recall    = |{s > 0} and {z > 0}| / |{z > 0}|   (true activations found)
  precision = |{s > 0} and {z > 0}| / |{s > 0}|   (predicted ones that fire)

with z = W x + b, the true pre-activation, and the predictor's bytes per token
(r d + f r) * pb against the up matrix's f d * wb.

This is a design aid for choosing the rank; nothing on the kernel path calls it.
"""
from __future__ import annotations

import numpy as np


def spectral_matrix(rng: np.random.Generator, f: int, d: int, alpha: float) -> np.ndarray:
    """W [f][d] = U diag(sigma) V^T with Haar-random U (f x d, orthonormal columns)
    and V (d x d), sigma_k = k^(-alpha) scaled so that the mean squared row norm is 1."""
    U, _ = np.linalg.qr(rng.standard_normal((f, d)))
    V, _ = np.linalg.qr(rng.standard_normal((d, d)))
    sigma = np.arange(1, d + 1, dtype=np.float64) ** (-float(alpha))
    sigma *= np.sqrt(f / np.sum(sigma ** 2))
    return (U * sigma) @ V.T


def rank_r_predictor(W: np.ndarray, r: int):
    """The rank-r truncated SVD of W as a predictor pair: A [r][d], B [f][r], B A = W_r."""
    U, s, Vt = np.linalg.svd(W, full_matrices=False)
    return s[:r, None] * Vt[:r], U[:, :r]


def predictor_quality(W: np.ndarray, bias: np.ndarray, A: np.ndarray, B: np.ndarray, X: np.ndarray) -> dict:
    """Recall and precision of mask (B A x + b > 0) against (W x + b > 0) over tokens X [n][d]."""
    Z = X @ W.T + bias
    S = (X @ A.T) @ B.T + bias
    truth, pred = Z > 0, S > 0
    tp = float(np.sum(truth & pred))
    return {"recall": tp / max(float(truth.sum()), 1.0), "precision": tp / max(float(pred.sum()), 1.0),
            "true_rate": float(truth.mean()), "predicted_rate": float(pred.mean())}


def study(d: int = 1024, f: int = 4096, ranks=(16, 64, 256, 1024), alphas=(0.0, 0.5, 1.0),
          p_mean: float = 0.1, tokens: int = 256, seed: int = 11, pb: float = 2.0, wb: float = 2.0) -> list:
    """One row per (alpha, rank): recall, precision, rates and the byte ratio.

    Firing probabilities are Zipf-like (p_k ~ 1/k, clamped to [0.01, 0.9], scaled to
    mean p_mean), and each neuron's bias is placed so that P(z_i > 0) = p_i for
    Gaussian x: b_i = Phi^-1(p_i) * |W_i|."""
    from scipy.special import ndtri

    rng = np.random.default_rng(seed)
    k = rng.permutation(f) + 1.0
    lo, hi = 1e-6, 1e6
    for _ in range(200):                           # bisection on the scale C of C / k
        c = np.sqrt(lo * hi)
        m = np.clip(c / k, 0.01, 0.9).mean()
        lo, hi = (c, hi) if m < p_mean else (lo, c)
    p = np.clip(np.sqrt(lo * hi) / k, 0.01, 0.9)
    X = rng.standard_normal((tokens, d))
    rows = []
    for alpha in alphas:
        W = spectral_matrix(rng, f, d, alpha)
        bias = ndtri(p) * np.linalg.norm(W, axis=1)
        U, s, Vt = np.linalg.svd(W, full_matrices=False)
        for r in ranks:
            r = min(int(r), d)
            A, B = s[:r, None] * Vt[:r], U[:, :r]
            q = predictor_quality(W, bias, A, B, X)
            q.update(alpha=float(alpha), rank=r, predictor_bytes=(r * d + f * r) * pb,
                     byte_ratio=(r * d + f * r) * pb / (f * d * wb))
            rows.append(q)
    return rows


def table(rows) -> str:
    out = ["| spectrum alpha | rank | predictor / up bytes | true rate | predicted rate | recall | precision |",
           "|---|---|---|---|---|---|---|"]
    for q in rows:
        out.append(f"| {q['alpha']:.1f} | {q['rank']} | {q['byte_ratio']:.3f} | {q['true_rate']:.3f} | "
                   f"{q['predicted_rate']:.3f} | {q['recall']:.3f} | {q['precision']:.3f} |")
    return "\n".join(out)
