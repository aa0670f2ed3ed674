"""Pins for the seeded workload generator (CPU only)."""
import json
import os

import numpy as np
import pytest
from scipy.special import ndtri as scipy_ndtri

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_philox_known_answers(gen):
    for row in _rows("philox4x32_10_kat.txt"):
        vals = [int(v, 16) for v in row]
        out = gen.philox4x32_10(vals[0:4], vals[4:6])
        assert [int(v) for v in out] == vals[6:10]


def test_ndtri_known_values(gen):
    for p, z in _rows("ndtri_points.txt"):
        got = gen.ndtri(np.array([float(p)]))[0]
        assert abs(got - float(z)) <= 4e-15 * max(1.0, abs(float(z))), (p, got, z)


def test_ndtri_matches_library_and_symmetry(gen):
    p = np.concatenate([np.geomspace(1e-300, 1e-3, 400), np.linspace(1e-3, 1 - 1e-3, 20001),
                        1 - np.geomspace(1e-16, 1e-3, 200)])
    got = gen.ndtri(p)
    ref = scipy_ndtri(p)
    assert np.all(np.abs(got - ref) <= 1e-14 * np.maximum(1.0, np.abs(ref)))
    q = np.arange(1, 2 ** 19 + 1, dtype=np.float64) / 2.0 ** 20      # dyadic: 1 - q is exact
    assert np.array_equal(gen.ndtri(q), -gen.ndtri(1 - q))
    assert gen.ndtri(np.array([0.5]))[0] == 0.0


def test_f16_rounding_matches_numpy(gen):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(400000) * np.exp(rng.uniform(-25, 12, 400000))
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25,
                     2.0 ** -14, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf])
    x = np.concatenate([x, edge, -edge])
    assert np.array_equal(gen.to_f16(x).view(np.uint16), x.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("f,target", [(2048, 0.10), (11008, 0.12), (28672, 0.20), (32768, 0.10),
                                      (49152, 0.08), (1000, 0.3)])
def test_zipf_mean_and_clamp(gen, f, target):
    p = gen.zipf_probs(1234, 0, f, target)
    assert abs(p.mean() - target) < 1e-9
    assert p.min() >= 0.01 and p.max() <= 0.9
    C = gen.zipf_constant(f, target)
    k = gen.zipf_ranks(1234, 0, f)
    assert np.array_equal(np.sort(k), np.arange(1, f + 1))        # a permutation of 1..f
    np.testing.assert_allclose(p, np.clip(C / k.astype(np.float64), 0.01, 0.9), rtol=1e-15, atol=0)
    # number of neurons at the upper clamp: k <= C / 0.9
    assert int(np.sum(p == 0.9)) == int(np.floor(C / 0.9))


def test_hot_first_perm(gen):
    p = gen.zipf_probs(99, 3, 4096, 0.1)
    perm = gen.hot_first_perm(p)
    ref = np.lexsort((np.arange(p.size), -p))         # p descending, id ascending
    assert np.array_equal(perm, ref)
    assert np.array_equal(np.sort(perm), np.arange(p.size))


def test_rows_keyed_by_original_id(gen):
    cfg = gen.CONFIGS[0].with_(d=256, ffn=300, rank=64)
    a = gen.make_layer(cfg, 0, order="hot_first")
    b = gen.make_layer(cfg, 0, order="identity")
    assert np.array_equal(a.up, b.up[a.perm])
    assert np.array_equal(a.downT, b.downT[a.perm])
    assert np.array_equal(a.B, b.B[a.perm])
    assert np.array_equal(a.bias, b.bias[a.perm])
    assert np.array_equal(a.A, b.A)


def test_gaussian_moments(gen):
    z = gen.gaussian_rows(5, 1, 0, None, 64, 20000, 1.0, "f64")
    assert abs(z.mean()) < 4 / np.sqrt(z.size)
    assert abs(z.var() - 1) < 4 * np.sqrt(2 / z.size)
    # fourth moment of a normal is 3
    assert abs((z ** 4).mean() - 3) < 0.05


def test_firing_probability_matches_target(gen):
    """w.x + b > 0 fires with probability p for x ~ N(0, I) (bias = PhiInv(p) * ||w||)."""
    cfg = gen.CONFIGS[0].with_(d=256, ffn=64, rank=64)
    lw = gen.make_layer(cfg, 0)
    X = gen.gaussian_rows(cfg.seed, 99, 0, None, 20000, cfg.d, 1.0, "f64")
    Z = X @ lw.up.astype(np.float64).T + lw.bias.astype(np.float64)[None, :]
    rate = (Z > 0).mean(axis=0)
    p = lw.p_storage
    sd = np.sqrt(p * (1 - p) / X.shape[0])
    assert np.all(np.abs(rate - p) < 5 * sd + 1e-3)


def test_q4_layer_bias_norm(gen):
    cfg = gen.CONFIGS[4].with_(d=256, ffn=128, rank=64)
    lw = gen.make_layer(cfg, 0)
    nib, sc = lw.up.nibbles, lw.up.scales
    assert nib.shape == (128, 128) and sc.shape == (128, 8)
    q = np.concatenate([nib & 15, nib >> 4], axis=1)   # order is irrelevant for a norm
    sq = ((q.astype(np.int64) - 8) ** 2).reshape(128, 2, 8, 16).sum(axis=(1, 3))
    norm = np.sqrt((sc.view(np.float16).astype(np.float64) ** 2 * sq).sum(axis=1))
    np.testing.assert_allclose(gen.row_norms(lw.up), norm, rtol=1e-14)
    # every nibble value appears, uniformly
    counts = np.bincount(q.ravel(), minlength=16)
    assert counts.min() > 0.8 * q.size / 16


def test_fig8_fixture_is_readable():
    with open(os.path.join(GOLDEN, "fig8_fixture.json")) as fh:
        fx = json.load(fh)
    assert fx["ffn"] == 8 and fx["skipped_hot"] == [7]


def test_hot_count_follows_the_byte_model(gen):
    """The prefix ends at the first slot whose p is below 1 - r pb / (n_in d wb)."""
    cfg = gen.CONFIGS[4]                       # Q4_0 ReLU: 1 - 1024*2 / (12288 * 18/32)
    p_min = 1.0 - cfg.rank * 2.0 / (cfg.d * 18.0 / 32.0)
    ps = np.array([0.9, 0.8, p_min + 1e-9, p_min - 1e-9, 0.9, 0.1])
    assert gen.hot_count(cfg, ps) == 3
    assert gen.hot_count(cfg, np.array([0.1, 0.9])) == 0
    assert gen.hot_count(cfg, np.array([0.95, 0.99])) == 2
    c1 = gen.CONFIGS[1]                        # ReGLU fp16: two input rows per neuron
    assert gen.hot_count(c1, np.array([1.0 - 1024 * 2.0 / (2 * 4096 * 2.0) + 1e-9, 0.0])) == 1
