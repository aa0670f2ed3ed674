"""Python binding of the C ABI in include/pi.h (libpi.so, HIP for gfx950).

Argument marshalling only: every step of the sparse FFN runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  There is
no CPU fallback: if the shared library is missing or fails to load, importing
the binding's entry points raises.

Entry points (same names and meaning as the C functions):
  workspace_bytes(layers, batch)
  predict(layer, x, idx, count, scores=None, mask=None, ws=None)
  sparse_ffn(layer, x, idx, count, y, mask=None, ws=None)
  ffn_stack(layers, x, out, counts=None, trace=None, ws=None, nz_counts=None)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpi.so")

PI_OK, PI_EINVAL, PI_EUNSUPPORTED, PI_EWORKSPACE, PI_EHIP = 0, 1, 2, 3, 4
PI_F32, PI_F16, PI_Q4_0 = 0, 1, 2
PI_RELU, PI_REGLU, PI_RELU2 = 0, 1, 2

_DTYPE = {"f32": PI_F32, "f16": PI_F16, "q4_0": PI_Q4_0}
_ACT = {"relu": PI_RELU, "reglu": PI_REGLU, "relu2": PI_RELU2}


class PiError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = f" [{lib().pi_last_hip_error().decode()}]" if status == PI_EHIP else ""
        super().__init__(f"{where}: {status_str(status)} ({status}){detail}")
        self.status = status


class PiMat(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("scale", ctypes.c_void_p)]


class PiLayer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("ffn", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("act", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("p_dtype", ctypes.c_int32),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("pbias", ctypes.c_void_p), ("gate", PiMat), ("up", PiMat), ("downT", PiMat), ("b_down", ctypes.c_void_p),
                ("hot", ctypes.c_int32), ("dense_frac", ctypes.c_float)]


class PiTrace(ctypes.Structure):
    _fields_ = [("x_in", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("count", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32)]


# kernels of one layer, in the order the trace events bracket them
LAYER_KERNELS = {1: ("k_predict_t", "k_score", "k_down"),
                 2: ("k_bglue", "k_bpred1", "k_bsplit_t", "k_bscore", "k_compact", "k_bup", "k_bdown")}


# the layout of the structures above; the library must report the same version
ABI_VERSION = 6

_lib = None


def lib():
    """Load libpi.so (raises if it is not built, or built from another ABI version)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.pi_abi_version.restype = I32
        L.pi_status_str.argtypes = [ctypes.c_int]
        L.pi_status_str.restype = ctypes.c_char_p
        L.pi_workspace_bytes.argtypes = [P, I32, I32]
        L.pi_workspace_bytes.restype = SZ
        L.pi_predict.argtypes = [P, P, I32, P, P, P, P, P, SZ, P]
        L.pi_predict.restype = ctypes.c_int
        L.pi_sparse_ffn.argtypes = [P, P, I32, P, P, P, P, P, SZ, P]
        L.pi_sparse_ffn.restype = ctypes.c_int
        L.pi_ffn_stack.argtypes = [P, I32, P, I32, P, P, P, P, P, SZ, P]
        L.pi_ffn_stack.restype = ctypes.c_int
        L.pi_ffn_stack_static.argtypes = [P, I32, P, I32, P, P, P, P, P]
        L.pi_ffn_stack_static.restype = ctypes.c_int
        L.pi_last_hip_error.restype = ctypes.c_char_p
        got = int(L.pi_abi_version())
        if got != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {got}, this binding expects {ABI_VERSION} "
                               "(rebuild with __graft_entry__.build())")
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().pi_abi_version())


def status_str(s: int) -> str:
    return lib().pi_status_str(int(s)).decode()


def _p(t) -> Optional[int]:
    """Device address of a tensor (or an int address), None for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, where: str):
    if status != PI_OK:
        raise PiError(status, where)


# ------------------------------------------------------------------ layers
class DeviceLayer:
    """One layer's tensors resident on the GPU plus the matching pi_layer record."""

    def __init__(self, *, d, ffn, rank, act, w_dtype, p_dtype, A, B, bias, up, downT, gate=None,
                 b_down=None, pbias=None, hot=0, dense_frac=0.0):
        self.d, self.ffn, self.rank = int(d), int(ffn), int(rank)
        self.hot = int(hot)
        self.dense_frac = float(dense_frac)
        self.act, self.w_dtype, self.p_dtype = act, w_dtype, p_dtype
        self.A, self.B, self.bias, self.up, self.downT, self.gate, self.b_down = \
            A, B, bias, up, downT, gate, b_down
        self.pbias = pbias
        self.struct = self._make_struct()

    @staticmethod
    def _mat(m):
        if m is None:
            return PiMat(None, None)
        if isinstance(m, tuple):            # Q4_0: (nibbles, scales)
            return PiMat(m[0].data_ptr(), m[1].data_ptr())
        return PiMat(m.data_ptr(), None)

    def _make_struct(self) -> PiLayer:
        return PiLayer(self.d, self.ffn, self.rank, _ACT[self.act], _DTYPE[self.w_dtype],
                       _DTYPE[self.p_dtype], _p(self.A), _p(self.B), _p(self.bias),
                       _p(self.pbias), self._mat(self.gate), self._mat(self.up), self._mat(self.downT),
                       _p(self.b_down), self.hot, self.dense_frac)

    @classmethod
    def upload(cls, lw, device="cuda") -> "DeviceLayer":
        """Copy a host layer (numpy arrays; Q4_0 matrices with .nibbles/.scales) to the GPU."""
        import numpy as np
        import torch

        def t(a):
            if a is None:
                return None
            if hasattr(a, "nibbles"):
                nib = torch.from_numpy(np.ascontiguousarray(a.nibbles)).to(device)
                sc = torch.from_numpy(np.ascontiguousarray(a.scales).view(np.int16)).to(device)
                return (nib, sc)
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)

        cfg = lw.cfg
        return cls(d=cfg.d, ffn=cfg.ffn, rank=cfg.rank, act=cfg.act, w_dtype=cfg.w_dtype,
                   p_dtype=cfg.p_dtype, A=t(lw.A), B=t(lw.B), bias=t(lw.bias), up=t(lw.up),
                   downT=t(lw.downT), gate=t(lw.gate), b_down=t(lw.b_down),
                   pbias=t(getattr(lw, "pbias", None)), hot=int(getattr(lw, "hot", 0) or 0),
                   dense_frac=float(getattr(lw, "dense_frac", 0.0) or 0.0))

    def nbytes(self) -> int:
        tot = 0
        for m in (self.A, self.B, self.bias, self.pbias, self.up, self.downT, self.gate, self.b_down):
            if m is None:
                continue
            for x in (m if isinstance(m, tuple) else (m,)):
                tot += x.numel() * x.element_size()
        return tot


def _layer_array(layers: Sequence[DeviceLayer]):
    arr = (PiLayer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L.struct
    return arr


# ------------------------------------------------------------- entry points
def workspace_bytes(layers, batch: int = 1) -> int:
    layers = [layers] if isinstance(layers, DeviceLayer) else list(layers)
    arr = _layer_array(layers)
    return int(lib().pi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), len(layers), batch))


def alloc_workspace(layers, batch: int = 1, device="cuda"):
    import torch
    n = workspace_bytes(layers, batch)
    if n == 0:
        raise PiError(PI_EINVAL, "workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def predict(layer: DeviceLayer, x, idx, count, scores=None, mask=None, ws=None, batch: int = 1,
            stream=None):
    ws = alloc_workspace(layer, batch) if ws is None else ws
    st = lib().pi_predict(ctypes.byref(layer.struct), _p(x), batch, _p(scores), _p(mask), _p(idx),
                          _p(count), _p(ws), ws.numel(), _stream(stream))
    _check(st, "pi_predict")


def sparse_ffn(layer: DeviceLayer, x, idx, count, y, mask=None, ws=None, batch: int = 1,
               stream=None):
    ws = alloc_workspace(layer, batch) if ws is None else ws
    st = lib().pi_sparse_ffn(ctypes.byref(layer.struct), _p(x), batch, _p(idx), _p(count),
                             _p(mask), _p(y), _p(ws), ws.numel(), _stream(stream))
    _check(st, "pi_sparse_ffn")


def make_trace(n_layers: int, recs: Sequence[dict]):
    """Trace records; a record's optional "events" entry is a list of hipEvent_t handles
    (ints, e.g. from HipEvents) or objects with a .cuda_event handle."""
    arr = (PiTrace * n_layers)()
    keep = []
    for i, r in enumerate(recs):
        evs = r.get("events")
        if evs:
            ptrs = (ctypes.c_void_p * len(evs))(*[e if isinstance(e, int) else e.cuda_event for e in evs])
            keep.append(ptrs)
            ev_arg, n_ev = ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), len(evs)
        else:
            ev_arg, n_ev = None, 0
        arr[i] = PiTrace(_p(r.get("x_in")), _p(r.get("scores")), _p(r.get("mask")),
                         _p(r.get("idx")), _p(r.get("count")), _p(r.get("y")), ev_arg, n_ev)
    arr._keep = keep
    return arr


class Stack:
    """A stack of DeviceLayers with its layer array and workspace kept alive."""

    def __init__(self, layers: Sequence[DeviceLayer], batch: int = 1, ws=None):
        self.layers = list(layers)
        self.batch = batch
        self.arr = _layer_array(self.layers)
        self.ws = alloc_workspace(self.layers, batch) if ws is None else ws

    def __call__(self, x, out, counts=None, trace=None, stream=None, nz_counts=None):
        tr = None if trace is None else ctypes.cast(trace, ctypes.c_void_p)
        st = lib().pi_ffn_stack(ctypes.cast(self.arr, ctypes.c_void_p), len(self.layers), _p(x),
                                self.batch, _p(out), _p(counts), _p(nz_counts), tr, _p(self.ws),
                                self.ws.numel(), _stream(stream))
        _check(st, "pi_ffn_stack")


def ffn_stack(layers, x, out, counts=None, trace=None, ws=None, batch: int = 1, stream=None, nz_counts=None):
    Stack(layers, batch, ws)(x, out, counts, trace, stream, nz_counts)


STATIC_WORKSPACE_BYTES = 96 << 20   # PI_STATIC_WORKSPACE_BYTES


def ffn_stack_static(layers, x, out, counts=None, trace=None, batch: int = 1, stream=None, nz_counts=None):
    """pi_ffn_stack_static: the stack on the library's own per-GPU scratch array (no workspace)."""
    arr = _layer_array(list(layers))
    tr = None if trace is None else ctypes.cast(trace, ctypes.c_void_p)
    st = lib().pi_ffn_stack_static(ctypes.cast(arr, ctypes.c_void_p), len(arr), _p(x), batch, _p(out),
                                   _p(counts), _p(nz_counts), tr, _stream(stream))
    _check(st, "pi_ffn_stack_static")


# ------------------------------------------------------- HIP runtime plumbing
_hip = None


def hip_runtime():
    """The HIP runtime (libamdhip64) for graphs and timing events."""
    global _hip
    if _hip is None:
        H = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        H.hipGetErrorString.restype = ctypes.c_char_p
        H.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        H.hipEventDestroy.argtypes = [P]
        H.hipEventRecord.argtypes = [P, P]
        H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        H.hipStreamBeginCapture.argtypes = [P, ctypes.c_int]
        H.hipStreamEndCapture.argtypes = [P, ctypes.POINTER(P)]
        H.hipGraphInstantiate.argtypes = [ctypes.POINTER(P), P, P, P, ctypes.c_size_t]
        H.hipGraphLaunch.argtypes = [P, P]
        H.hipGraphExecDestroy.argtypes = [P]
        H.hipGraphDestroy.argtypes = [P]
        H.hipStreamCreate.argtypes = [ctypes.POINTER(P)]
        H.hipStreamDestroy.argtypes = [P]
        H.hipStreamSynchronize.argtypes = [P]
        _hip = H
    return _hip


def _hip_check(r: int, where: str):
    if r != 0:
        raise RuntimeError(f"{where}: {hip_runtime().hipGetErrorString(r).decode()} ({r})")


class HipEvent:
    """A timing hipEvent_t; int(ev) is the handle."""

    def __init__(self):
        self.h = ctypes.c_void_p()
        _hip_check(hip_runtime().hipEventCreate(ctypes.byref(self.h)), "hipEventCreate")

    def __int__(self):
        return int(self.h.value)

    def record(self, stream):
        _hip_check(hip_runtime().hipEventRecord(self.h, _stream(stream)), "hipEventRecord")

    def elapsed_ms(self, later: "HipEvent") -> float:
        ms = ctypes.c_float()
        _hip_check(hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self.h, later.h), "hipEventElapsedTime")
        return float(ms.value)

    def __del__(self):
        if _hip is not None and self.h:
            _hip.hipEventDestroy(self.h)


class HipStream:
    """A plain hipStream_t (default flags and priority); .cuda_stream is the handle."""

    def __init__(self):
        self.h = ctypes.c_void_p()
        _hip_check(hip_runtime().hipStreamCreate(ctypes.byref(self.h)), "hipStreamCreate")

    @property
    def cuda_stream(self) -> int:
        return int(self.h.value)

    def synchronize(self):
        _hip_check(hip_runtime().hipStreamSynchronize(self.h), "hipStreamSynchronize")

    def __del__(self):
        if _hip is not None and self.h:
            _hip.hipStreamDestroy(self.h)


class HipGraph:
    """Stream capture of fn(stream) into an instantiated hipGraph, replayed on that stream.

    Only library calls belong inside fn: nothing in it may allocate."""

    def __init__(self, stream, fn):
        H = hip_runtime()
        self.stream = _stream(stream)
        self.g, self.ge = ctypes.c_void_p(), ctypes.c_void_p()
        _hip_check(H.hipStreamBeginCapture(self.stream, 0), "hipStreamBeginCapture")  # global mode
        try:
            fn(stream)
        finally:
            _hip_check(H.hipStreamEndCapture(self.stream, ctypes.byref(self.g)), "hipStreamEndCapture")
        _hip_check(H.hipGraphInstantiate(ctypes.byref(self.ge), self.g, None, None, 0), "hipGraphInstantiate")

    def replay(self):
        _hip_check(hip_runtime().hipGraphLaunch(self.ge, self.stream), "hipGraphLaunch")

    def __del__(self):
        if _hip is not None:
            if self.ge:
                _hip.hipGraphExecDestroy(self.ge)
            if self.g:
                _hip.hipGraphDestroy(self.g)


EXPORTED = ("pi_workspace_bytes", "pi_predict", "pi_sparse_ffn", "pi_ffn_stack", "pi_ffn_stack_static",
            "pi_status_str", "pi_abi_version", "pi_last_hip_error")
