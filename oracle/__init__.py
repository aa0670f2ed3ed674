"""CPU oracle for the predictor-guided, neuron-aware sparse FFN (PowerInfer).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The GPU library never imports it, and it imports nothing from the
GPU library: the two share no code, no kernels, no helpers and no constants.
Both consume the same seeded input arrays from ``workload``.

Plain, slow, obviously correct: every quantity is computed in float64 with
NumPy, straight from its definition, in the order the pages describe it.  A
matrix-vector product (``@``) is a library primitive and is used as one step.

What it computes (per layer, per sequence b, x_b in R^d):

  predictor   t = A x ;  s_i = c_i + sum_j B[i,j] t_j            (``predictor_scores``)
      A low-rank MLP predicts which FFN neurons of the current layer will
      fire (GeekNews summary, "CPU/GPUハイブリッド推論方式": adaptive predictor;
      unite.ai article, "Online-Phase" and "Adaptive Sparsity-Prädiktoren";
      机器之心 article, Fig. 8 paragraph).  Reading taken: the hidden layer is
      the identity (a rank-r GEMV pair); the output bias c_i is the layer's
      ``pbias`` when given, else the up/gate bias b_i (``predictor_bias``).
  threshold   m_i = (float32(s_i) > 0), strict; NaN is inactive   (``threshold``)
      The pages give no threshold; 0 is the centre of the reported
      ambiguity band.  The decision is taken on the score rounded to float32,
      the precision the GPU takes it in; rounding never changes the sign of a
      non-zero double.
  hot prefix  m_i = 1 for storage slots i < hot, whatever s_i is     (``hot_prefix``)
      Optional (hot = 0: off).  The hottest neurons are placed first by the
      hot-first permutation and computed for every token without a
      prediction -- the on-GPU form of the pages' hot/cold neuron split
      (PowerInfer repository README, hot-activated neurons; unite.ai article,
      "Neuronen-Platzierung und -Verwaltung"; 机器之心 article, hot/cold
      paragraph).  Where the predictor would have switched such a neuron off,
      its h = act(.) is added anyway, so the result changes there.
  list        ascending storage ids i with m_i = 1 (union over b)  (``active_list``)
      Only neuron ids are listed; weights are never converted into a sparse
      format (unite.ai, "Neuronenbewusster Operator").
  activation  ReLU:  h_i = max(b_i + W_up[i] . x, 0)
              ReGLU: h_i = max(b_i + W_gate[i] . x, 0) * (W_up[i] . x)
              Squared ReLU: h_i = max(b_i + W_up[i] . x, 0)^2
      (GeekNews summary: ReLU / ReGLU / Squared ReLU models), computed only for
      listed neurons with m_{b,i} = 1; a neuron in the union but not in
      sequence b's own mask contributes h = 0 for b.
  down        y = sum_{i listed, m_{b,i}} h_i * W_downT[i]  (+ b_down)
      Rows of the up/gate matrices and columns of the down matrix of active
      neurons only (unite.ai, "Online-Phase": individual neuron rows and
      columns).  W_downT row i is column i of W_down.
  glue        v = x + y ;  x' = v / sqrt(mean(v^2) + 1e-6)        (``rms_glue``)
      Not on the pages: a residual plus parameter-free RMS norm so that a
      stack of layers keeps its firing rates.

Storage order is whatever order the rows are given in (hot-first in the
workloads); the unite.ai article's neuron tables map storage slots back to
original neuron ids ("Neuronen-Platzierung und -Verwaltung").

Q4_0 rows are (nibbles uint8 [rows][d/2], scales binary16 [rows][d/32]):
weight j of a 32-block is the low nibble of byte j (j < 16) or the high
nibble of byte j - 16 (j >= 16), and w = scale * (q - 8).
"""
from __future__ import annotations

import numpy as np

EPS_GLUE = 1e-6


# --------------------------------------------------------------------- decode
def _is_q4(m) -> bool:
    return hasattr(m, "nibbles") and hasattr(m, "scales")


def q4_decode(nibbles: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Q4_0 rows to float64: w = scale * (q - 8), nibble order as in the module doc."""
    nibbles = np.asarray(nibbles, dtype=np.uint8)
    rows, half = nibbles.shape
    nblk = half // 16
    blocks = nibbles.reshape(rows, nblk, 16)
    q = np.empty((rows, nblk, 32), dtype=np.int64)
    q[:, :, :16] = blocks & 0x0F          # weights 0..15: low nibbles
    q[:, :, 16:] = blocks >> 4            # weights 16..31: high nibbles
    d = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    w = d[:, :, None] * (q - 8).astype(np.float64)
    return w.reshape(rows, nblk * 32)


def decode(m) -> np.ndarray:
    """Whole matrix to float64 (float32 and binary16 convert exactly)."""
    if _is_q4(m):
        return q4_decode(m.nibbles, m.scales)
    return np.asarray(m).astype(np.float64)


def decode_rows(m, rows) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    if _is_q4(m):
        return q4_decode(m.nibbles[rows], m.scales[rows])
    return np.asarray(m)[rows].astype(np.float64)


# ------------------------------------------------------------------ predictor
def predictor_scores(A, B, bias, X) -> np.ndarray:
    """s[b, i] = bias_i + sum_j B[i, j] * (sum_k A[j, k] * X[b, k]), float64 [nb][ffn]."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    A64 = decode(A)
    B64 = decode(B)
    T = X @ A64.T                      # t = A x, one row per sequence
    return T @ B64.T + np.asarray(bias, dtype=np.float64)[None, :]


def threshold(S) -> np.ndarray:
    """m = float32(s) > 0 (strict; zero and NaN are inactive)."""
    return np.asarray(S, dtype=np.float64).astype(np.float32) > 0


def active_list(mask_1d) -> np.ndarray:
    """Ascending ids i with mask[i] set, written out as a plain scan."""
    out = []
    for i, m in enumerate(np.asarray(mask_1d, dtype=bool).tolist()):
        if m:
            out.append(i)
    return np.asarray(out, dtype=np.int64)


def hot_prefix(masks, hot: int) -> np.ndarray:
    """Masks with the first ``hot`` storage slots on in every sequence."""
    M = np.array(np.atleast_2d(masks), dtype=bool, copy=True)
    M[:, :int(hot)] = True
    return M


def union_mask(masks) -> np.ndarray:
    masks = np.atleast_2d(np.asarray(masks, dtype=bool))
    u = np.zeros(masks.shape[1], dtype=bool)
    for row in masks:
        u = u | row
    return u


# ------------------------------------------------------------------------ FFN
def _act(act: str, zg: np.ndarray, zu: np.ndarray | None) -> np.ndarray:
    """The activation of a neuron from its pre-activation(s).

    The GeekNews summary's model list names ReLU, ReGLU and Squared ReLU
    (ReLU-family activations, the ones with exact zeros).  Their textbook
    forms: ReLU max(z, 0); ReGLU max(z_gate, 0) * z_up; Squared ReLU
    max(z, 0)^2, which is zero exactly where ReLU is."""
    if act == "relu":
        return np.maximum(zg, 0.0)
    if act == "reglu":
        return np.maximum(zg, 0.0) * zu
    if act == "relu2":
        r = np.maximum(zg, 0.0)
        return r * r
    raise ValueError(act)


def _uses_gate(act: str) -> bool:
    """ReGLU gates with its own matrix; ReLU and Squared ReLU use the up matrix alone."""
    return act == "reglu"


def sparse_ffn(act, gate, up, downT, bias, X, masks, b_down=None) -> np.ndarray:
    """y[b] from the rows of the neurons in sequence b's own mask only, float64 [nb][d].

    ReLU and Squared ReLU use ``up`` with ``bias``; ReGLU uses ``gate`` with
    ``bias`` and ``up`` without bias.  Contributions are summed in ascending
    neuron id.
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    masks = np.atleast_2d(np.asarray(masks, dtype=bool))
    bias = np.asarray(bias, dtype=np.float64)
    nb, d = X.shape
    Y = np.zeros((nb, d), dtype=np.float64)
    for b in range(nb):
        idx = active_list(masks[b])
        if idx.size:
            x = X[b]
            if not _uses_gate(act):
                zg = decode_rows(up, idx) @ x + bias[idx]
                zu = None
            else:
                zg = decode_rows(gate, idx) @ x + bias[idx]
                zu = decode_rows(up, idx) @ x
            h = _act(act, zg, zu)
            D = decode_rows(downT, idx)
            y = np.zeros(d, dtype=np.float64)
            for j in range(idx.size):     # ascending neuron order
                y += h[j] * D[j]
            Y[b] = y
        if b_down is not None:
            Y[b] += np.asarray(b_down, dtype=np.float64)
    return Y


def dense_ffn(act, gate, up, downT, bias, X, masks=None, b_down=None) -> np.ndarray:
    """Dense FFN over every neuron, y = W_down (m * act(W x + b)); m = all ones if None."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    bias = np.asarray(bias, dtype=np.float64)
    U = decode(up)
    D = decode(downT)
    if not _uses_gate(act):
        ZG = X @ U.T + bias[None, :]
        ZU = None
    else:
        ZG = X @ decode(gate).T + bias[None, :]
        ZU = X @ U.T
    H = _act(act, ZG, ZU)
    if masks is not None:
        H = H * np.atleast_2d(np.asarray(masks, dtype=bool))
    Y = H @ D
    if b_down is not None:
        Y = Y + np.asarray(b_down, dtype=np.float64)[None, :]
    return Y


def rms_glue(X, Y, eps: float = EPS_GLUE) -> np.ndarray:
    """x' = v / sqrt(mean(v^2) + eps), v = x + y, per sequence, float64."""
    V = np.atleast_2d(np.asarray(X, dtype=np.float64)) + np.atleast_2d(np.asarray(Y, dtype=np.float64))
    ms = (V * V).mean(axis=1, keepdims=True)
    return V / np.sqrt(ms + eps)


# ------------------------------------------------------------- layer / stack
def _get(layer, name):
    if layer is None:
        return None
    return layer.get(name) if isinstance(layer, dict) else getattr(layer, name, None)


def predictor_bias(layer):
    """The predictor's output bias c: the layer's ``pbias`` when it has one,
    else the up/gate bias b (the predictor "plus bias b_i" of the workloads
    whose rows have unit norm)."""
    pbias = _get(layer, "pbias")
    return _get(layer, "bias") if pbias is None else pbias


def ffn_bias(layer):
    """The bias of the gate (ReGLU) or up (ReLU, Squared ReLU) projection, b."""
    return _get(layer, "bias")


def layer_forward(layer, X, act: str | None = None) -> dict:
    """One layer for a batch of sequences X [nb][d].

    Returns scores (float64), masks (per sequence), the ascending union list,
    its count and y (float64).  A layer with ``hot`` > 0 has its first ``hot``
    neurons on without a prediction (their scores are still returned).
    """
    act = act or _get(layer, "act") or _get(_get(layer, "cfg"), "act")
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    S = predictor_scores(_get(layer, "A"), _get(layer, "B"), predictor_bias(layer), X)
    M = threshold(S)
    hot = int(_get(layer, "hot") or 0)
    if hot:
        M = hot_prefix(M, hot)
    idx = active_list(union_mask(M))
    Y = sparse_ffn(act, _get(layer, "gate"), _get(layer, "up"), _get(layer, "downT"),
                   ffn_bias(layer), X, M, _get(layer, "b_down"))
    return {"x_in": X, "scores": S, "masks": M, "idx": idx, "count": int(idx.size), "y": Y}


def stack_forward(layers, X0, act: str | None = None) -> dict:
    """Stack of layers with the residual RMS glue between them; out = x_L."""
    X = np.atleast_2d(np.asarray(X0, dtype=np.float64))
    recs = []
    for layer in layers:
        r = layer_forward(layer, X, act)
        X = rms_glue(X, r["y"])
        r["x_out"] = X
        recs.append(r)
    return {"layers": recs, "out": X}


def macs_per_token(d: int, ffn: int, rank: int, n_mat: int, active: float) -> float:
    """Multiply-adds per token and layer at a given number of active neurons."""
    return rank * d + ffn * rank + active * n_mat * d
