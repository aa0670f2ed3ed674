"""The layer-local replay used by the GPU parity tests, exercised on the CPU.

A float32 trace of a stack is written out here from the oracle's own steps
(what a correct GPU run would record), and the replay must accept it.  Then
one defect at a time is planted in a copy of that trace -- a wrong y in a
deep layer, a mask bit flipped outside the band, a wrong glue, a wrong list --
and the replay must reject it, including after an earlier layer in which a
neuron inside the band was decided the other way.
"""
import copy

import numpy as np
import pytest

import oracle
from parity import BAND, replay_stack


def fake_trace(host, x0, act):
    """Per-layer records as the GPU library writes them (float32), from the oracle."""
    X = np.asarray(x0, np.float32)
    recs = []
    for h in host:
        S = oracle.predictor_scores(h.A, h.B, oracle.predictor_bias(h), X.astype(np.float64))
        s32 = S.astype(np.float32)
        M = s32 > 0
        Y = oracle.sparse_ffn(act, h.gate, h.up, h.downT, oracle.ffn_bias(h), X.astype(np.float64), M)
        y32 = Y.astype(np.float32)
        idx = np.flatnonzero(M.any(axis=0)).astype(np.int32)
        full = np.full(S.shape[1], -1, np.int32)
        full[:idx.size] = idx
        recs.append(dict(x_in=X.copy(), scores=s32, mask=M.astype(np.uint8), idx=full, count=int(idx.size),
                         y=y32))
        X = oracle.rms_glue(X.astype(np.float64), y32.astype(np.float64)).astype(np.float32)
    return recs, X


@pytest.fixture(scope="module")
def stack(gen):
    cfg = gen.CONFIGS[3].with_(d=256, ffn=700, rank=64, n_layers=4)
    host = [gen.make_layer(cfg, l) for l in range(cfg.n_layers)]
    x0 = gen.make_x(cfg, 2, seqs=3)
    recs, out = fake_trace(host, x0, cfg.act)
    return cfg, host, x0, recs, out


def test_replay_accepts_a_correct_trace(stack):
    cfg, host, x0, recs, out = stack
    st = replay_stack(host, recs, out, x0, "f16", cfg.act)
    assert st["layers"] == 4 and st["max_y_err"] < 1e-6 and st["max_glue_err"] < 1e-6


def _fails(host, recs, out, x0, act):
    try:
        replay_stack(host, recs, out, x0, "f16", act)
    except AssertionError:
        return True
    return False


def test_replay_rejects_a_wrong_y_in_the_last_layer(stack):
    cfg, host, x0, recs, out = stack
    bad = copy.deepcopy(recs)
    j = int(np.argmax(np.abs(bad[3]["y"][1])))
    bad[3]["y"][1, j] *= 1.01                     # 1% of max|y|: far above the 1e-4 tolerance
    assert _fails(host, bad, out, x0, cfg.act)


def test_replay_rejects_a_mask_flip_outside_the_band(stack):
    cfg, host, x0, recs, out = stack
    bad = copy.deepcopy(recs)
    S = bad[2]["scores"][0].astype(np.float64)
    i = int(np.argmax(np.abs(S)))                 # the neuron farthest from the threshold
    bad[2]["mask"][0, i] ^= 1
    bad[2]["scores"][0, i] = -bad[2]["scores"][0, i]
    assert _fails(host, bad, out, x0, cfg.act)


def test_replay_rejects_a_wrong_glue(stack):
    cfg, host, x0, recs, out = stack
    bad = copy.deepcopy(recs)
    bad[2]["x_in"][0] = bad[2]["x_in"][0] * np.float32(1.001)
    assert _fails(host, bad, out, x0, cfg.act)
    bad_out = out.copy()
    bad_out[2, 5] += 0.01
    assert _fails(host, recs, bad_out, x0, cfg.act)


def test_replay_rejects_a_wrong_list(stack):
    cfg, host, x0, recs, out = stack
    bad = copy.deepcopy(recs)
    bad[1]["count"] -= 1
    assert _fails(host, bad, out, x0, cfg.act)
    bad = copy.deepcopy(recs)
    c = bad[1]["count"]
    bad[1]["idx"][[0, c - 1]] = bad[1]["idx"][[c - 1, 0]]   # not ascending
    assert _fails(host, bad, out, x0, cfg.act)


def test_replay_keeps_gating_after_a_band_flip(stack):
    """A band neuron decided the other way in layer 0 changes every later input; the
    replay follows the changed trajectory and still catches a defect in layer 3."""
    cfg, host, x0, recs, out = stack
    # push one score of layer 0 into the band and flip its decision, as a GPU may
    h0 = host[0]
    X = np.asarray(x0, np.float64)
    S = oracle.predictor_scores(h0.A, h0.B, oracle.predictor_bias(h0), X)
    i = int(np.argmin(np.abs(S[0])))
    h0b = copy.copy(h0)
    c = np.asarray(oracle.predictor_bias(h0), np.float32).copy()
    c[i] -= np.float32(S[0, i] - BAND / 4)       # oracle score of neuron i now +BAND/4
    h0b.pbias = c
    hb = [h0b] + host[1:]
    recs_b, out_b = fake_trace(hb, x0, cfg.act)
    # the "GPU" took neuron i as inactive (score just below zero) in layer 0
    r0 = recs_b[0]
    assert r0["mask"][0, i] == 1
    r0["mask"][0, i] = 0
    r0["scores"][0, i] = -np.float32(BAND / 8)
    idx = np.flatnonzero(r0["mask"].astype(bool).any(axis=0)).astype(np.int32)
    r0["idx"][:] = -1
    r0["idx"][:idx.size] = idx
    r0["count"] = int(idx.size)
    # recompute the rest of the trajectory from that decision
    Xl = r0["x_in"]
    r0["y"] = oracle.sparse_ffn(cfg.act, h0b.gate, h0b.up, h0b.downT, oracle.ffn_bias(h0b),
                                Xl.astype(np.float64), r0["mask"].astype(bool)).astype(np.float32)
    x1 = oracle.rms_glue(Xl.astype(np.float64), r0["y"].astype(np.float64)).astype(np.float32)
    tail, out2 = fake_trace(hb[1:], x1, cfg.act)
    good = [r0] + tail
    st = replay_stack(hb, good, out2, x0, "f16", cfg.act)
    assert st["band_flips"] >= 1
    bad = copy.deepcopy(good)
    j = int(np.argmax(np.abs(bad[3]["y"][0])))
    bad[3]["y"][0, j] *= 1.01
    assert _fails(hb, bad, out2, x0, cfg.act)
