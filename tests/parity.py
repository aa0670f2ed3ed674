"""Comparison protocol between the GPU library and the CPU oracle.

The predictor's threshold turns floating point into a decision, so where the
oracle's float64 score lies within BAND of 0 both outcomes are correct; those
neurons are counted, never failed.  Everything else is exact:
  - scores: max |s_gpu - s_oracle| < BAND (so every neuron outside the band
    has the same sign on both sides);
  - masks: bit-exact outside the band;
  - lists: the GPU list equals the ascending list of the GPU's own mask and
    the count equals its length;
  - outputs: max |y_gpu - y_oracle| <= tol * max |y_oracle| on the same mask.

Stacks are checked by layer-local replay: for every layer and sequence, the
oracle takes the GPU's own layer input x_l and the GPU's own mask, recomputes
the scores and y_l, and then the glue from x_l and the GPU's y_l, which must
give the GPU's next layer input (or the stack output).  A neuron decided
differently inside the band therefore never hides a later layer from the
check (the prediction is made per layer: unite.ai article, "Online-Phase").
The end-to-end output from x_0 is compared too and reported, not gated.
"""
from __future__ import annotations

import numpy as np

import oracle

BAND = 1e-4

# Output tolerances, relative to max |y_oracle|.  fp32 weights: 1e-5 (the
# stated bar).  fp16 and Q4_0 weights at batch 1: every weight is exact in
# fp32 and products accumulate in fp32 over at most d (12288) terms per dot
# and a few thousand rows per output, so the error is ~1e-5 of max|y|; 1e-4
# keeps a 10x margin and is 100x tighter than the stated 1e-2, tight enough
# that one dropped neuron (~1/sqrt(k) of rms y) fails it.
TOL = {"f32": 1e-5, "f16": 1e-4, "q4_0": 1e-4}


def check_scores_masks(S_or, scores, mask, band=BAND):
    """One sequence: S_or float64 [f], scores float32 [f], mask uint8/bool [f]."""
    S_or = np.asarray(S_or, np.float64)
    m_gpu = np.asarray(mask).astype(bool)
    st = {}
    if scores is not None:
        err = np.abs(np.asarray(scores, np.float64) - S_or)
        st["max_score_err"] = float(err.max()) if err.size else 0.0
        assert st["max_score_err"] < band, st
        # the GPU's mask is the GPU's own score's sign
        assert np.array_equal(m_gpu, np.asarray(scores, np.float32) > 0)
    m_or = oracle.threshold(S_or)
    inband = np.abs(S_or) < band
    differ = m_or != m_gpu
    assert not (differ & ~inband).any(), np.flatnonzero(differ & ~inband)[:10]
    st["band"] = int(inband.sum())
    st["band_flips"] = int((differ & inband).sum())
    return st


def check_list(mask, idx, count):
    m = np.asarray(mask).astype(bool)
    count = int(count)
    assert count == int(m.sum()), (count, int(m.sum()))
    assert np.array_equal(np.asarray(idx)[:count], np.flatnonzero(m))


def check_nz_count(layer, act, x_in, mask, nz, rel_band=1e-5):
    """Rows of W_down^T read at batch 1: active neurons whose h is nonzero.

    h != 0 exactly when the gate (ReGLU) or up (ReLU) pre-activation is > 0
    (and, for ReGLU, the up product is nonzero).  The pre-activation z is
    recomputed in float64 on the GPU's own layer input; neurons with |z|
    within rel_band of max |z| may go either way."""
    rows = np.flatnonzero(np.asarray(mask).astype(bool))
    x = np.asarray(x_in, np.float64)
    w = layer.gate if act == "reglu" else layer.up
    z = oracle.decode_rows(w, rows) @ x + np.asarray(layer.bias, np.float64)[rows]
    if act == "reglu":
        zu = oracle.decode_rows(layer.up, rows) @ x
        z = np.where(zu == 0.0, -np.abs(z), z)
    tol = rel_band * (float(np.abs(z).max()) if z.size else 0.0)
    lo, hi = int((z > tol).sum()), int((z > -tol).sum())
    assert lo <= int(nz) <= hi, (int(nz), lo, hi)
    return hi - lo


def rel_err(y, y_ref):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    scale = float(np.abs(y_ref).max()) if y_ref.size else 0.0
    err = float(np.abs(y - y_ref).max()) if y_ref.size else 0.0
    return err / scale if scale > 0 else err


def check_y(y, y_ref, tol):
    assert np.all(np.isfinite(y))
    e = rel_err(y, y_ref)
    assert e <= tol, (e, tol)
    return e


# The stack glue, x' = rms(x + y), in float32 on the GPU against float64 here:
# one rounding of v = x + y, a float32 sum of d squares and a reciprocal square
# root, each a few units in the last place (~1e-7 relative); 1e-5 of max |x'|
# bounds them with margin and still fails a dropped term of v.
GLUE_TOL = 1e-5


def _rows(a):
    return np.atleast_2d(np.asarray(a))


def replay_stack(host, trace, out, x0, w_dtype, act, band=BAND, end_to_end=True, seqs=None, score_units=None):
    """Layer-local replay of a stack run.

    host: the layers (workload.LayerWeights); trace: per-layer dicts of numpy
    arrays from the GPU -- x_in [nb][d], scores [nb][ffn], mask [nb][ffn],
    idx [ffn], count, y [nb][d] and, at batch 1, nz (rows of W_down^T read);
    out: the GPU's stack output [nb][d]; x0: the stack input [nb][d].
    Every layer is gated, for every sequence or for the sequences in `seqs`
    (the union list is always checked against every sequence's mask).
    score_units[l] (default 1) is the unit in which layer l's scores are
    compared with the band: a layer fed with inputs of another magnitude has
    scores of that magnitude.  A layer with a hot-dense prefix (``hot`` > 0)
    must have its first ``hot`` mask bytes set; their scores are not written by
    the GPU and are not compared.  Returns statistics.
    """
    tol = TOL[w_dtype]
    X0 = _rows(x0).astype(np.float32)
    sel = np.arange(X0.shape[0]) if seqs is None else np.asarray(sorted(seqs))
    st = {"layers": len(host), "band": 0, "band_flips": 0, "max_score_err": 0.0, "max_y_err": 0.0,
          "max_glue_err": 0.0, "nz_ambiguous": 0}
    assert np.array_equal(_rows(trace[0]["x_in"]), X0), "the first layer's input is the stack input"
    for l, (h, g) in enumerate(zip(host, trace)):
        # the union list, against every sequence's mask
        check_list(_rows(g["mask"]).astype(bool).any(axis=0), g["idx"], g["count"])
        X = _rows(g["x_in"])[sel].astype(np.float64)
        scores, mask, yg = _rows(g["scores"])[sel], _rows(g["mask"])[sel], _rows(g["y"])[sel]
        assert np.all(np.isfinite(X)) and np.all(np.isfinite(yg))
        # predictor and threshold on the GPU's own layer input
        S = oracle.predictor_scores(h.A, h.B, oracle.predictor_bias(h), X)
        u = 1.0 if score_units is None else float(score_units[l])
        hot = int(getattr(h, "hot", 0) or 0)
        assert np.all(mask[:, :hot] == 1), "the hot prefix is on in every sequence"
        for b in range(X.shape[0]):
            s = check_scores_masks(S[b, hot:] / u, scores[b, hot:].astype(np.float64) / u, mask[b, hot:], band)
            st["band"] += s["band"]
            st["band_flips"] += s["band_flips"]
            st["max_score_err"] = max(st["max_score_err"], s["max_score_err"])
        if "nz" in g:
            st["nz_ambiguous"] += check_nz_count(h, act, X[0], mask[0], g["nz"])
        # y on the GPU's own input and mask
        Y = oracle.sparse_ffn(act, h.gate, h.up, h.downT, oracle.ffn_bias(h), X, mask.astype(bool),
                              getattr(h, "b_down", None))
        for b in range(X.shape[0]):
            st["max_y_err"] = max(st["max_y_err"], check_y(yg[b], Y[b], tol))
        # the glue of the GPU's own x and y gives the next layer's input
        Xn = oracle.rms_glue(X, yg)
        nxt = _rows(trace[l + 1]["x_in"] if l + 1 < len(trace) else out)[sel]
        for b in range(X.shape[0]):
            st["max_glue_err"] = max(st["max_glue_err"], check_y(nxt[b], Xn[b], GLUE_TOL))
    if end_to_end:
        ref = oracle.stack_forward(host, X0[sel])
        o = _rows(out)[sel]
        st["out_err_end_to_end"] = max(rel_err(o[b], ref["out"][b]) for b in range(o.shape[0]))
    return st
