"""Seeded synthetic workloads for the predictor-guided sparse FFN.

This module builds inputs only (weights, biases, firing probabilities, the
hot-first storage order, token vectors).  It contains none of the method's
arithmetic and is shared, as input data, by the CPU oracle (``oracle/``) and
the GPU library (``activation_sparse_predict_amd``), neither of which it
imports.

The workload model follows the PowerInfer pages' observation that neuron
activation follows a power law: a few hot neurons fire for most inputs, many
cold neurons fire input-dependently (GeekNews summary, "PowerInferが解決しよう
としている問題"; unite.ai article, introduction; 机器之心 article, "PowerInfer
架构").  Neuron i fires with target probability p_i from a Zipf law over a
seeded random rank order, and its bias is placed so that the pre-activation
is positive with exactly that probability for x ~ N(0, I).  Storage order is
hot-first (p descending, ties by original id), the on-GPU analogue of the
neuron tables that map each neuron to its original matrix position (unite.ai
article, "Neuronen-Platzierung und -Verwaltung").

Layouts (row-major, storage order = hot-first unless ``order="identity"``):
  A      [rank][d]     predictor first matrix      (p_dtype)
  B      [ffn][rank]   predictor second matrix     (p_dtype)
  bias   [ffn]         float32; gate bias (ReGLU) or up bias (ReLU):
                       PhiInv(p_i) * ||stored row_i||, so w_i.x + b_i > 0 with
                       probability p_i for x ~ N(0, I)
  pbias  [ffn]         float32 or None; the predictor's own output bias.
                       None (the predictor adds the up/gate bias b_i) for
                       fp32/fp16 weights, whose rows have norm ~1, so that
                       b_i ~ PhiInv(p_i).  Q4_0 rows have norm ~37 (scale
                       8|N(0, 1/d)| times q - 8 with q uniform), so b_i would
                       mark only ~3% of the neurons instead of the configured
                       8%; there pbias = PhiInv(p_i): the predictor output
                       B_i.(A x) has unit variance for x ~ N(0, I)
                       (A ~ N(0, 1/d), B ~ N(0, 1/r)), so c_i marks neuron i
                       with probability ~p_i
  gate   [ffn][d]      ReGLU only                  (w_dtype)
  up     [ffn][d]                                  (w_dtype)
  downT  [ffn][d]      row i = column i of W_down  (w_dtype)
Q4_0 matrices are a pair (nibbles uint8 [ffn][d/2], scales uint16 [ffn][d/32]);
within a 32-weight block, weight j < 16 is the low nibble of byte j and weight
j + 16 the high nibble of byte j, and w = scale * (q - 8).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.cpp")
_LIB = os.path.join(_HERE, "libpigen.so")

TAG_A, TAG_B, TAG_GATE, TAG_UP, TAG_DOWN, TAG_X, TAG_ZIPF = 1, 2, 3, 4, 5, 6, 7
TAG_SCALE = 16  # added to a matrix tag for its Q4_0 scales

DT_F32, DT_F16, DT_F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the generator (host C++, g++)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        c = ctypes
        P = c.c_void_p
        L.pg_philox4x32_10.argtypes = [P, P, P]
        L.pg_ndtri.argtypes = [c.c_double]
        L.pg_ndtri.restype = c.c_double
        L.pg_ndtri_vec.argtypes = [P, c.c_int64, P]
        L.pg_f64_to_f16.argtypes = [P, c.c_int64, P]
        L.pg_zipf_constant.argtypes = [c.c_int64, c.c_double, c.c_double, c.c_double, c.c_double]
        L.pg_zipf_constant.restype = c.c_double
        L.pg_zipf_ranks.argtypes = [c.c_uint32, c.c_uint32, c.c_uint32, c.c_int64, P]
        L.pg_zipf_probs.argtypes = [c.c_uint32, c.c_uint32, c.c_uint32, c.c_int64, c.c_double,
                                    c.c_double, c.c_double, c.c_double, P]
        L.pg_zipf_probs.restype = c.c_double
        L.pg_hot_first_perm.argtypes = [P, c.c_int64, P]
        L.pg_gaussian_rows.argtypes = [c.c_uint32, c.c_uint32, c.c_uint32, P, c.c_int64, c.c_int64,
                                       c.c_double, c.c_int, P, c.c_int]
        L.pg_random_bytes_rows.argtypes = [c.c_uint32, c.c_uint32, c.c_uint32, P, c.c_int64,
                                           c.c_int64, P, c.c_int]
        L.pg_q4_scales_rows.argtypes = [c.c_uint32, c.c_uint32, c.c_uint32, P, c.c_int64,
                                        c.c_int64, c.c_double, c.c_double, P, c.c_int]
        L.pg_row_norms.argtypes = [P, P, c.c_int64, c.c_int64, c.c_int, P, c.c_int]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ------------------------------------------------------------------ primitives
def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().pg_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def ndtri(p) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.float64)
    out = np.empty_like(p)
    lib().pg_ndtri_vec(_ptr(p), p.size, _ptr(out))
    return out


def to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().pg_f64_to_f16(_ptr(x), x.size, _ptr(out))
    return out.view(np.float16)


def zipf_constant(f: int, target: float, s: float = 1.0, lo: float = 0.01, hi: float = 0.9) -> float:
    return lib().pg_zipf_constant(f, s, lo, hi, target)


def zipf_ranks(seed: int, layer: int, f: int) -> np.ndarray:
    out = np.empty(f, dtype=np.int32)
    lib().pg_zipf_ranks(seed, TAG_ZIPF, layer, f, _ptr(out))
    return out


def zipf_probs(seed: int, layer: int, f: int, target: float, s: float = 1.0, lo: float = 0.01,
               hi: float = 0.9) -> np.ndarray:
    out = np.empty(f, dtype=np.float64)
    lib().pg_zipf_probs(seed, TAG_ZIPF, layer, f, s, lo, hi, target, _ptr(out))
    return out


def hot_first_perm(p: np.ndarray) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.float64)
    out = np.empty(p.size, dtype=np.int32)
    lib().pg_hot_first_perm(_ptr(p), p.size, _ptr(out))
    return out


def gaussian_rows(seed: int, tag: int, layer: int, row_ids: Optional[np.ndarray], nrows: int,
                  ncols: int, stddev: float, dtype: str, nthreads: int = 0) -> np.ndarray:
    code, npdt = {"f32": (DT_F32, np.float32), "f16": (DT_F16, np.uint16),
                  "f64": (DT_F64, np.float64)}[dtype]
    out = np.empty((nrows, ncols), dtype=npdt)
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int32)
    lib().pg_gaussian_rows(seed, tag, layer, _ptr(ids), nrows, ncols, stddev, code, _ptr(out),
                           nthreads)
    return out.view(np.float16) if dtype == "f16" else out


def q4_rows(seed: int, tag: int, layer: int, row_ids: Optional[np.ndarray], nrows: int, ncols: int,
            scale_std: float, scale_mult: float = 8.0, nthreads: int = 0):
    assert ncols % 32 == 0
    nib = np.empty((nrows, ncols // 2), dtype=np.uint8)
    sc = np.empty((nrows, ncols // 32), dtype=np.uint16)
    ids = None if row_ids is None else np.ascontiguousarray(row_ids, dtype=np.int32)
    lib().pg_random_bytes_rows(seed, tag, layer, _ptr(ids), nrows, ncols // 2, _ptr(nib), nthreads)
    lib().pg_q4_scales_rows(seed, tag + TAG_SCALE, layer, _ptr(ids), nrows, ncols // 32, scale_std,
                            scale_mult, _ptr(sc), nthreads)
    return Q4Matrix(nib, sc)


def row_norms(mat, nthreads: int = 0) -> np.ndarray:
    if isinstance(mat, Q4Matrix):
        nrows, ncols = mat.nibbles.shape[0], mat.nibbles.shape[1] * 2
        out = np.empty(nrows, dtype=np.float64)
        lib().pg_row_norms(_ptr(mat.nibbles), _ptr(mat.scales), nrows, ncols, 3, _ptr(out), nthreads)
        return out
    nrows, ncols = mat.shape
    code = {np.dtype(np.float32): 0, np.dtype(np.float16): 1}[mat.dtype]
    out = np.empty(nrows, dtype=np.float64)
    lib().pg_row_norms(_ptr(mat.view(np.uint16) if code == 1 else mat), None, nrows, ncols, code,
                       _ptr(out), nthreads)
    return out


# ------------------------------------------------------------------ data model
@dataclass
class Q4Matrix:
    nibbles: np.ndarray  # uint8 [rows][cols/2]
    scales: np.ndarray   # uint16 (binary16 bits) [rows][cols/32]

    @property
    def shape(self):
        return (self.nibbles.shape[0], self.nibbles.shape[1] * 2)

    def take_rows(self, rows):
        return Q4Matrix(self.nibbles[rows], self.scales[rows])


@dataclass(frozen=True)
class FFNConfig:
    name: str
    d: int
    ffn: int
    rank: int
    n_layers: int
    act: str          # "relu" | "reglu" | "relu2" (Squared ReLU)
    w_dtype: str      # "f32" | "f16" | "q4_0"
    p_dtype: str      # "f32" | "f16"
    mean_active: float
    seed: int
    batches: tuple = (1,)
    tokens: int = 128
    zipf_s: float = 1.0
    p_lo: float = 0.01
    p_hi: float = 0.9

    def with_(self, **kw) -> "FFNConfig":
        return replace(self, **kw)


_SEED0 = 0x50490000

CONFIGS = {
    0: FFNConfig("relu-fp32 d512 f2048 r64", 512, 2048, 64, 1, "relu", "f32", "f32", 0.10,
                 _SEED0 + 0, (1,), 16),
    1: FFNConfig("llama2-7b-shaped reglu-fp16 d4096 f11008 r1024 L32", 4096, 11008, 1024, 32,
                 "reglu", "f16", "f16", 0.12, _SEED0 + 1, (1,), 128),
    2: FFNConfig("opt-30b-shaped relu-fp16 d7168 f28672 r1024 L48", 7168, 28672, 1024, 48, "relu",
                 "f16", "f16", 0.20, _SEED0 + 2, (1,), 128),
    3: FFNConfig("falcon-40b-shaped relu-fp16 d8192 f32768 r1024 L60", 8192, 32768, 1024, 60,
                 "relu", "f16", "f16", 0.10, _SEED0 + 3, (1, 8, 32), 128),
    4: FFNConfig("opt-175b-shaped relu-q4_0 d12288 f49152 r1024 L96", 12288, 49152, 1024, 96,
                 "relu", "q4_0", "f16", 0.08, _SEED0 + 4, (1, 32), 128),
}


@dataclass
class LayerWeights:
    cfg: FFNConfig
    layer: int
    p: np.ndarray          # float64 [ffn], ORIGINAL order
    perm: np.ndarray       # int32 [ffn], storage slot -> original id
    A: np.ndarray          # [rank][d]
    B: np.ndarray          # [ffn][rank], storage order
    bias: np.ndarray       # float32 [ffn], storage order
    up: object             # ndarray [ffn][d] or Q4Matrix
    downT: object
    gate: object = None    # ReGLU only
    b_down: Optional[np.ndarray] = None
    pbias: Optional[np.ndarray] = None   # float32 [ffn], storage order
    hot: int = 0                         # hot-dense prefix length (storage slots [0, hot))
    dense_frac: float = 0.0              # batched FFN over every neuron from this union fraction (0: default)

    @property
    def p_storage(self) -> np.ndarray:
        return self.p[self.perm]

    def nbytes(self) -> int:
        def nb(m):
            if m is None:
                return 0
            if isinstance(m, Q4Matrix):
                return m.nibbles.nbytes + m.scales.nbytes
            return m.nbytes
        return sum(nb(m) for m in (self.A, self.B, self.bias, self.pbias, self.up, self.downT,
                                   self.gate))


def make_layer(cfg: FFNConfig, layer: int, order: str = "hot_first", nthreads: int = 0,
               p_override: Optional[np.ndarray] = None) -> LayerWeights:
    d, f, r = cfg.d, cfg.ffn, cfg.rank
    p = zipf_probs(cfg.seed, layer, f, cfg.mean_active, cfg.zipf_s, cfg.p_lo, cfg.p_hi) \
        if p_override is None else np.ascontiguousarray(p_override, dtype=np.float64)
    if order == "hot_first":
        perm = hot_first_perm(p)
    elif order == "identity":
        perm = np.arange(f, dtype=np.int32)
    else:
        raise ValueError(order)
    sd = 1.0 / np.sqrt(d)
    A = gaussian_rows(cfg.seed, TAG_A, layer, None, r, d, sd, cfg.p_dtype, nthreads)
    B = gaussian_rows(cfg.seed, TAG_B, layer, perm, f, r, 1.0 / np.sqrt(r), cfg.p_dtype, nthreads)

    def mat(tag):
        if cfg.w_dtype == "q4_0":
            return q4_rows(cfg.seed, tag, layer, perm, f, d, sd, 8.0, nthreads)
        return gaussian_rows(cfg.seed, tag, layer, perm, f, d, sd, cfg.w_dtype, nthreads)

    gate = mat(TAG_GATE) if cfg.act == "reglu" else None
    up = mat(TAG_UP)
    downT = mat(TAG_DOWN)
    norms = row_norms(gate if cfg.act == "reglu" else up, nthreads)
    z = ndtri(p[perm])
    bias = (z * norms).astype(np.float32)
    # the predictor adds b_i where it is on the predictor's scale (rows of norm
    # ~1), and its own PhiInv(p_i) where it is not (Q4_0 rows, norm ~37)
    pbias = z.astype(np.float32) if cfg.w_dtype == "q4_0" else None
    return LayerWeights(cfg, layer, p, perm, A, B, bias, up, downT, gate, None, pbias)


def make_x(cfg: FFNConfig, token: int, seqs: int = 1, stream: int = 0) -> np.ndarray:
    """Token vectors x ~ N(0, I), float32 [seqs][d], keyed by (token, sequence)."""
    ids = np.arange(seqs, dtype=np.int32) + np.int32(stream * 4096)
    return gaussian_rows(cfg.seed, TAG_X, token, ids, seqs, cfg.d, 1.0, "f32")


def make_tokens(cfg: FFNConfig, n_tokens: int, seqs: int = 1, first: int = 0) -> np.ndarray:
    """float32 [n_tokens][seqs][d]."""
    return np.stack([make_x(cfg, first + t, seqs) for t in range(n_tokens)])


def hot_count(cfg: FFNConfig, p_storage: np.ndarray) -> int:
    """Length of a hot-dense prefix for a layer: the leading storage slots
    (hot-first order) whose firing probability makes computing them for every
    token cheaper in bytes than predicting them.  Predicted, neuron i costs its
    row of B (r * pb bytes) and, with probability p_i, its up/gate rows
    (n_in * d * wb); computed for every token it costs those rows always (the
    down row is read only when h != 0, either way).  So the prefix holds the
    neurons with n_in * d * wb * (1 - p_i) < r * pb."""
    pb = 4.0 if cfg.p_dtype == "f32" else 2.0
    wb = {"f32": 4.0, "f16": 2.0, "q4_0": 18.0 / 32.0}[cfg.w_dtype]
    n_in = 2 if cfg.act == "reglu" else 1
    p_min = 1.0 - cfg.rank * pb / (n_in * cfg.d * wb)
    ps = np.asarray(p_storage, dtype=np.float64)
    below = np.flatnonzero(ps < p_min)
    return int(below[0]) if below.size else int(ps.size)
