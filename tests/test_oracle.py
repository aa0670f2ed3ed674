"""Pins for the CPU oracle (CPU only).

Each test ties the oracle to something other than itself: exact rational
arithmetic on tiny inputs, closed forms, invariants of the method, a library
routine for the compaction, and the worked example of the pages (Fig. 8).
The planted-mistake tests at the end swap a deliberately wrong step into the
oracle and check that one of these pins catches it.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class Q4:
    def __init__(self, nibbles, scales):
        self.nibbles, self.scales = nibbles, scales


def tiny_layer(rng, d, f, r, act="relu", scale=1.0, pbias=False):
    """Small float64-exact layer (values are dyadic rationals, exact in float32).

    With pbias, the predictor gets an output bias of its own, drawn apart from
    the up/gate bias (and of the opposite sign wherever they would coincide)."""
    def m(*shape):
        return (rng.integers(-64, 65, size=shape) / 32.0 * scale).astype(np.float32)
    L = dict(act=act, A=m(r, d), B=m(f, r), bias=m(f), up=m(f, d), downT=m(f, d),
             gate=m(f, d) if act == "reglu" else None, b_down=None)
    if pbias:
        c = m(f)
        c[c == L["bias"]] = -L["bias"][c == L["bias"]] + np.float32(0.5)
        L["pbias"] = c
    return L


# ---------------------------------------------------------------- exact brute force
def frac_layer(L, x):
    """The layer in exact rational arithmetic, following the definitions step by step
    (with a hot-dense prefix: slots i < L["hot"] are on whatever their score)."""
    A, B, bias = L["A"], L["B"], L["bias"]
    # the predictor's own output bias c where the layer has one, else b
    c = L.get("pbias") if L.get("pbias") is not None else bias
    d = A.shape[1]
    r, f = A.shape[0], B.shape[0]
    X = [Fraction(float(v)) for v in x]
    t = [sum(Fraction(float(A[j, k])) * X[k] for k in range(d)) for j in range(r)]
    s = [Fraction(float(c[i])) + sum(Fraction(float(B[i, j])) * t[j] for j in range(r))
         for i in range(f)]
    hot = int(L.get("hot", 0) or 0)
    m = [i < hot or v > 0 for i, v in enumerate(s)]
    y = [Fraction(0)] * d
    for i in range(f):
        if not m[i]:
            continue
        if L["act"] in ("relu", "relu2"):
            z = Fraction(float(bias[i])) + sum(Fraction(float(L["up"][i, k])) * X[k] for k in range(d))
            h = max(z, Fraction(0))
            if L["act"] == "relu2":       # Squared ReLU
                h = h * h
        else:
            g = Fraction(float(bias[i])) + sum(Fraction(float(L["gate"][i, k])) * X[k] for k in range(d))
            u = sum(Fraction(float(L["up"][i, k])) * X[k] for k in range(d))
            h = max(g, Fraction(0)) * u
        for k in range(d):
            y[k] += h * Fraction(float(L["downT"][i, k]))
    return s, m, y


@pytest.mark.parametrize("pbias", [False, True], ids=["shared_bias", "own_pbias"])
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_matches_exact_rationals(act, seed, pbias):
    rng = np.random.default_rng(seed)
    d, f, r = 12, 10, 5                   # all different, so a transposed operand cannot pass
    L = tiny_layer(rng, d, f, r, act, pbias=pbias)
    x = (rng.integers(-64, 65, size=d) / 16.0).astype(np.float32)
    s_ex, m_ex, y_ex = frac_layer(L, x)
    out = oracle.layer_forward(L, x[None, :])
    np.testing.assert_allclose(out["scores"][0], [float(v) for v in s_ex], rtol=0, atol=1e-12)
    assert out["masks"][0].tolist() == m_ex
    assert out["idx"].tolist() == [i for i in range(f) if m_ex[i]]
    assert out["count"] == sum(m_ex)
    y_ref = np.array([float(v) for v in y_ex])
    np.testing.assert_allclose(out["y"][0], y_ref, rtol=0, atol=1e-11 * max(1.0, np.abs(y_ref).max()))
    assert 0 < out["count"] < f            # the case exercises both branches


# ------------------------------------------------------------------- predictor
def test_predictor_zero_weights_gives_bias():
    rng = np.random.default_rng(3)
    f, r, d = 40, 8, 16
    bias = rng.standard_normal(f).astype(np.float32)
    S = oracle.predictor_scores(np.zeros((r, d), np.float32), np.zeros((f, r), np.float32), bias,
                                rng.standard_normal((3, d)))
    assert np.array_equal(S, np.broadcast_to(bias.astype(np.float64), (3, f)))
    assert np.array_equal(oracle.threshold(S)[0], bias > 0)


def test_predictor_identity_first_matrix_is_plain_gemv():
    rng = np.random.default_rng(4)
    d, f = 24, 50
    B = rng.standard_normal((f, d)).astype(np.float32)
    bias = rng.standard_normal(f).astype(np.float32)
    x = rng.standard_normal(d)
    S = oracle.predictor_scores(np.eye(d, dtype=np.float32), B, bias, x[None, :])[0]
    ref = np.array([sum(float(B[i, k]) * x[k] for k in range(d)) + float(bias[i]) for i in range(f)])
    np.testing.assert_allclose(S, ref, rtol=1e-13, atol=1e-13)


def test_threshold_is_strict_and_nan_inactive():
    s = np.array([1e-300, 0.0, -0.0, -1e-300, np.nan, np.inf, -np.inf, 1e-46, 2e-45])
    # float32(1e-300) == 0 and float32(1e-46) == 0: the decision is taken in float32
    assert oracle.threshold(s).tolist() == [False, False, False, False, False, True, False, False, True]


# ------------------------------------------------------------------ compaction
def test_active_list_matches_library():
    rng = np.random.default_rng(5)
    for f in [0, 1, 7, 64, 1000, 4097]:
        for p in [0.0, 0.05, 0.5, 1.0]:
            m = rng.random(f) < p
            assert np.array_equal(oracle.active_list(m), np.flatnonzero(m))


def test_union_list():
    M = np.array([[1, 0, 0, 1, 0], [0, 0, 1, 1, 0]], dtype=bool)
    assert oracle.active_list(oracle.union_mask(M)).tolist() == [0, 2, 3]


# ------------------------------------------------------------------------- FFN
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
def test_sparse_equals_dense_masked_and_all_ones_equals_dense(act):
    rng = np.random.default_rng(6)
    d, f = 64, 96
    L = tiny_layer(rng, d, f, 8, act)
    X = rng.standard_normal((4, d))
    M = rng.random((4, f)) < 0.3
    ys = oracle.sparse_ffn(act, L["gate"], L["up"], L["downT"], L["bias"], X, M)
    yd = oracle.dense_ffn(act, L["gate"], L["up"], L["downT"], L["bias"], X, M)
    np.testing.assert_allclose(ys, yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())
    ones = np.ones((4, f), dtype=bool)
    ya = oracle.sparse_ffn(act, L["gate"], L["up"], L["downT"], L["bias"], X, ones)
    yf = oracle.dense_ffn(act, L["gate"], L["up"], L["downT"], L["bias"], X)
    np.testing.assert_allclose(ya, yf, rtol=1e-12, atol=1e-12 * np.abs(yf).max())


def test_inactive_and_negative_neurons_contribute_exactly_zero():
    rng = np.random.default_rng(7)
    d, f = 32, 40
    L = tiny_layer(rng, d, f, 8, "relu")
    x = rng.standard_normal((1, d))
    M = rng.random((1, f)) < 0.5
    y0 = oracle.sparse_ffn("relu", None, L["up"], L["downT"], L["bias"], x, M)
    up2, down2 = L["up"].copy(), L["downT"].copy()
    up2[~M[0]] = np.nan                        # poisoned inactive rows are never read
    down2[~M[0]] = np.nan
    y1 = oracle.sparse_ffn("relu", None, up2, down2, L["bias"], x, M)
    assert np.array_equal(y0, y1)
    # neurons with z <= 0 contribute exactly 0: scaling their down rows changes nothing
    z = x[0] @ L["up"].astype(np.float64).T + L["bias"]
    down3 = L["downT"].copy()
    down3[z <= 0] *= 1000
    y2 = oracle.sparse_ffn("relu", None, L["up"], down3, L["bias"], x, M)
    assert np.array_equal(y0, y2)


def test_identity_closed_forms():
    rng = np.random.default_rng(8)
    d = 48
    I = np.eye(d, dtype=np.float32)
    x = rng.standard_normal((2, d))
    M = rng.random((2, d)) < 0.5
    y = oracle.sparse_ffn("relu", None, I, I, np.zeros(d, np.float32), x, M)
    assert np.array_equal(y, M * np.maximum(x, 0))
    y = oracle.sparse_ffn("reglu", I, 2 * I, I, np.zeros(d, np.float32), x, M)
    assert np.array_equal(y, M * np.maximum(x, 0) * 2 * x)
    b = np.full(d, 0.25, np.float32)
    y = oracle.sparse_ffn("relu", None, I, I, b, x, M)
    assert np.array_equal(y, M * np.maximum(x + 0.25, 0))
    # Squared ReLU: the square of the ReLU closed form
    y = oracle.sparse_ffn("relu2", None, I, I, np.zeros(d, np.float32), x, M)
    assert np.array_equal(y, M * np.maximum(x, 0) ** 2)


def test_permutation_invariance(gen):
    cfg = gen.CONFIGS[1].with_(d=256, ffn=320, rank=64, n_layers=1)
    a = gen.make_layer(cfg, 0, order="hot_first")
    b = gen.make_layer(cfg, 0, order="identity")
    X = gen.make_tokens(cfg, 3)[:, 0, :]
    ra, rb = oracle.layer_forward(a, X), oracle.layer_forward(b, X)
    np.testing.assert_allclose(ra["scores"], rb["scores"][:, a.perm], rtol=0, atol=1e-12)
    assert np.array_equal(ra["masks"], rb["masks"][:, a.perm])
    assert np.array_equal(np.sort(a.perm[ra["idx"]]), rb["idx"])
    np.testing.assert_allclose(ra["y"], rb["y"], rtol=0, atol=1e-12 * np.abs(rb["y"]).max())


def test_batch_invariance(gen):
    cfg = gen.CONFIGS[3].with_(d=256, ffn=512, rank=64, n_layers=1)
    lw = gen.make_layer(cfg, 0)
    X = gen.make_x(cfg, 0, seqs=8)
    rb = oracle.layer_forward(lw, X)
    for s in range(8):
        r1 = oracle.layer_forward(lw, X[s:s + 1])
        assert np.array_equal(r1["y"][0], rb["y"][s])
        assert np.array_equal(r1["masks"][0], rb["masks"][s])
    assert np.array_equal(rb["idx"], np.flatnonzero(rb["masks"].any(axis=0)))
    assert rb["count"] > max(oracle.layer_forward(lw, X[s:s + 1])["count"] for s in range(8))


def test_fig8_worked_example():
    with open(os.path.join(GOLDEN, "fig8_fixture.json")) as fh:
        fx = json.load(fh)
    f, d, r = fx["ffn"], 4, 2
    active = set(fx["predicted_active"])
    hot = fx["hot_neurons"]
    # hot neurons first (in id order), then the rest: storage slot -> original id
    perm = np.array(hot + [i for i in range(f) if i not in hot], dtype=np.int64)
    bias_orig = np.array([1.0 if i in active else -1.0 for i in range(f)], np.float32)
    rng = np.random.default_rng(9)
    up_orig = rng.standard_normal((f, d)).astype(np.float32)
    down_orig = rng.standard_normal((f, d)).astype(np.float32)
    L = dict(act="relu", A=np.zeros((r, d), np.float32), B=np.zeros((f, r), np.float32),
             bias=bias_orig[perm], up=up_orig[perm], downT=down_orig[perm], gate=None, b_down=None)
    x = rng.standard_normal((1, d))
    out = oracle.layer_forward(L, x)
    listed = sorted(perm[out["idx"]].tolist())
    assert listed == fx["predicted_active"]
    assert 7 not in listed and all(h in perm[:3] for h in fx["hot_neurons"])
    # the result is the contributions of the predicted neurons only
    y_ref = np.zeros(d)
    for i in fx["predicted_active"]:
        h = max(float(up_orig[i].astype(np.float64) @ x[0] + bias_orig[i]), 0.0)
        y_ref += h * down_orig[i].astype(np.float64)
    np.testing.assert_allclose(out["y"][0], y_ref, rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------- Q4_0
def test_q4_decode_special_values_and_nibble_order():
    scale = np.float16(0.375)
    for q, expect in [(8, 0.0), (0, -8 * 0.375), (15, 7 * 0.375)]:
        nib = np.full((1, 16), q | (q << 4), np.uint8)
        w = oracle.q4_decode(nib, np.array([[scale.view(np.uint16)]]))
        assert np.all(w == expect)
    # element j < 16 is the low nibble of byte j; element j + 16 its high nibble
    lo = np.arange(16, dtype=np.uint8)
    hi = (15 - np.arange(16)).astype(np.uint8)
    nib = (lo | (hi << 4)).astype(np.uint8)[None, :]
    w = oracle.q4_decode(nib, np.array([[np.float16(1.0).view(np.uint16)]]))[0]
    assert w[:16].tolist() == (lo.astype(float) - 8).tolist()
    assert w[16:].tolist() == (hi.astype(float) - 8).tolist()


def test_q4_pack_unpack_roundtrip():
    rng = np.random.default_rng(10)
    q = rng.integers(0, 16, size=(5, 64))
    sc = (np.abs(rng.standard_normal((5, 2))) + 0.1).astype(np.float16)
    blocks = q.reshape(5, 2, 32)
    nib = (blocks[:, :, :16] | (blocks[:, :, 16:] << 4)).astype(np.uint8).reshape(5, 32)
    w = oracle.q4_decode(nib, sc.view(np.uint16))
    np.testing.assert_array_equal(w, (sc.astype(np.float64).repeat(32, axis=1)) * (q - 8))


def test_q4_layer_matches_float_layer(gen):
    """A Q4_0 layer gives the same result as the same weights written out in float64."""
    cfg = gen.CONFIGS[4].with_(d=128, ffn=96, rank=64)
    lw = gen.make_layer(cfg, 0)
    X = gen.make_x(cfg, 0)
    Lf = dict(act="relu", A=lw.A, B=lw.B, bias=lw.bias, pbias=lw.pbias, gate=None, b_down=None,
              up=oracle.decode(lw.up), downT=oracle.decode(lw.downT))
    r1, r2 = oracle.layer_forward(lw, X), oracle.layer_forward(Lf, X)
    assert np.array_equal(r1["y"], r2["y"]) and np.array_equal(r1["idx"], r2["idx"])


# ---------------------------------------------------------------------- glue
def test_glue_closed_form():
    x = np.full((1, 16), 3.0)
    y = np.zeros((1, 16))
    np.testing.assert_allclose(oracle.rms_glue(x, y), 3.0 / np.sqrt(9.0 + 1e-6), rtol=1e-15)
    x = np.array([[1.0, -1.0, 2.0, -2.0]])
    y = np.array([[1.0, 1.0, 0.0, 0.0]])                # v = (2, 0, 2, -2), mean v^2 = 3
    np.testing.assert_allclose(oracle.rms_glue(x, y), np.array([[2, 0, 2, -2]]) / np.sqrt(3 + 1e-6),
                               rtol=1e-15)


def test_stack_chains_layers(gen):
    cfg = gen.CONFIGS[0].with_(d=128, ffn=256, rank=32, n_layers=3)
    layers = [gen.make_layer(cfg, l) for l in range(3)]
    X = gen.make_x(cfg, 0)
    out = oracle.stack_forward(layers, X)
    x = X.astype(np.float64)
    for l in range(3):
        r = oracle.layer_forward(layers[l], x)
        x = oracle.rms_glue(x, r["y"])
        assert np.array_equal(out["layers"][l]["y"], r["y"])
    assert np.array_equal(out["out"], x)


# ------------------------------------------------------------ planted mistakes
def _mutants():
    def no_bias(A, B, bias, X):
        X = np.atleast_2d(np.asarray(X, dtype=np.float64))
        return (X @ oracle.decode(A).T) @ oracle.decode(B).T

    def transposed_A(A, B, bias, X):
        X = np.atleast_2d(np.asarray(X, dtype=np.float64))
        A64 = oracle.decode(A)
        T = X[:, :A64.shape[0]] @ A64[:, :A64.shape[0]]
        return T @ oracle.decode(B).T + np.asarray(bias, dtype=np.float64)

    def nonstrict_threshold(S):
        return np.asarray(S, dtype=np.float64).astype(np.float32) >= 0

    def wrong_sign_threshold(S):
        return np.asarray(S, dtype=np.float64).astype(np.float32) < 0

    def off_by_one_list(mask_1d):
        return np.flatnonzero(np.asarray(mask_1d, bool)[1:]) + 1

    def relu_on_up(act, zg, zu):
        if act == "reglu":
            return zg * np.maximum(zu, 0.0)
        r = np.maximum(zg, 0.0)
        return r * r if act == "relu2" else r

    def relu2_not_squared(act, zg, zu):
        return np.maximum(zg, 0.0) if act in ("relu", "relu2") else np.maximum(zg, 0.0) * zu

    def pbias_ignored(layer):
        return oracle._get(layer, "bias")

    def pbias_in_the_ffn(layer):
        pb = oracle._get(layer, "pbias")
        return oracle._get(layer, "bias") if pb is None else pb

    def glue_no_residual(X, Y, eps=1e-6):
        V = np.atleast_2d(np.asarray(Y, dtype=np.float64))
        return V / np.sqrt((V * V).mean(axis=1, keepdims=True) + eps)

    return [("predictor_scores", no_bias), ("predictor_scores", transposed_A),
            ("threshold", nonstrict_threshold), ("threshold", wrong_sign_threshold),
            ("active_list", off_by_one_list), ("_act", relu_on_up), ("_act", relu2_not_squared),
            ("rms_glue", glue_no_residual), ("predictor_bias", pbias_ignored),
            ("ffn_bias", pbias_in_the_ffn)]


@pytest.mark.parametrize("name,fn", _mutants(), ids=lambda v: getattr(v, "__name__", str(v)))
def test_planted_mistake_is_caught(monkeypatch, gen, name, fn):
    monkeypatch.setattr(oracle, name, fn)
    pins = [lambda: test_layer_matches_exact_rationals("relu", 0, False),
            lambda: test_layer_matches_exact_rationals("reglu", 1, False),
            lambda: test_layer_matches_exact_rationals("relu2", 2, False),
            lambda: test_layer_matches_exact_rationals("relu", 0, True),
            lambda: test_layer_matches_exact_rationals("reglu", 1, True),
            test_predictor_zero_weights_gives_bias,
            test_threshold_is_strict_and_nan_inactive,
            test_active_list_matches_library,
            test_fig8_worked_example,
            test_glue_closed_form,
            test_identity_closed_forms]
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin catches the planted mistake in {name}"


# -------------------------------------------------------------- hot-dense prefix
@pytest.mark.parametrize("act", ["relu", "reglu", "relu2"])
@pytest.mark.parametrize("seed", [0, 1])
def test_hot_prefix_matches_exact_rationals(act, seed):
    """Slots [0, hot) are on without a prediction; the tail follows the threshold.
    The case is drawn so that the prefix holds a neuron the predictor switches off
    whose activation is non-zero, i.e. the prefix changes y."""
    rng = np.random.default_rng(100 + seed)
    d, f, r = 12, 10, 5
    for _ in range(200):
        L = tiny_layer(rng, d, f, r, act)
        x = (rng.integers(-64, 65, size=d) / 16.0).astype(np.float32)
        L["hot"] = 4
        s_ex, m_ex, y_ex = frac_layer(L, x)
        plain = dict(L, hot=0)
        _, m_plain, y_plain = frac_layer(plain, x)
        if m_plain[:4] != [True] * 4 and y_ex != y_plain and any(m_plain[4:]) and not all(m_plain[4:]):
            break
    else:
        pytest.skip("no case with a changed y found")
    out = oracle.layer_forward(L, x[None, :])
    np.testing.assert_allclose(out["scores"][0], [float(v) for v in s_ex], rtol=0, atol=1e-12)
    assert out["masks"][0].tolist() == m_ex
    assert out["masks"][0][:4].all()
    assert out["idx"].tolist() == [i for i in range(f) if m_ex[i]]
    y_ref = np.array([float(v) for v in y_ex])
    np.testing.assert_allclose(out["y"][0], y_ref, rtol=0, atol=1e-11 * max(1.0, np.abs(y_ref).max()))


def test_hot_prefix_over_every_neuron_is_the_dense_ffn():
    """hot = ffn: every neuron is on, so y is the dense FFN (a plain product over all
    neurons), whatever the predictor says."""
    rng = np.random.default_rng(7)
    d, f, r = 16, 24, 8
    L = tiny_layer(rng, d, f, r, "reglu")
    L["hot"] = f
    X = rng.standard_normal((3, d))
    out = oracle.layer_forward(L, X)
    assert out["masks"].all() and out["count"] == f
    dense = oracle.dense_ffn("reglu", L["gate"], L["up"], L["downT"], L["bias"], X)
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-12)
