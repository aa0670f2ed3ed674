"""The C ABI library loads, exports every declared symbol, and validates on the host.

No compute call is made here: every call below is rejected by host-side
validation before anything is enqueued, so the tests run without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pi():
    import activation_sparse_predict_amd as pi
    if not os.path.exists(pi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build_library()
    pi.lib()
    return pi


def declared_functions():
    with open(os.path.join(ROOT, "include", "pi.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"\b(pi_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["pi_predict", "pi_sparse_ffn", "pi_ffn_stack", "pi_workspace_bytes", "pi_status_str",
              "pi_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(pi):
    L = pi.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(pi.EXPORTED) <= set(declared_functions())


def test_abi_version_and_status_strings(pi):
    assert pi.abi_version() == 6
    # the binding's version is the header's
    hdr = open(os.path.join(ROOT, "include", "pi.h")).read()
    assert re.search(r"#define PI_ABI_VERSION (\d+)", hdr).group(1) == str(pi.ABI_VERSION) == "6"
    assert pi.status_str(0) == "ok"
    assert "workspace" in pi.status_str(3)


FAKE = 1 << 20  # a 16-byte-aligned fake device address; never dereferenced


def make_layer(pi, **kw):
    base = dict(d=512, ffn=1000, rank=64, act=pi.PI_RELU, w_dtype=pi.PI_F16, p_dtype=pi.PI_F16)
    base.update(kw)
    L = pi.PiLayer(base["d"], base["ffn"], base["rank"], base["act"], base["w_dtype"],
                   base["p_dtype"], FAKE, FAKE, FAKE, None, pi.PiMat(None, None), pi.PiMat(FAKE, None),
                   pi.PiMat(FAKE, None), None, base.get("hot", 0), base.get("dense_frac", 0.0))
    for k in ("gate", "up", "downT"):
        if k in kw:
            setattr(L, k, kw[k])
    for k in ("A", "B", "bias", "pbias", "b_down"):
        if k in kw:
            setattr(L, k, kw[k])
    return L


def ws_bytes(pi, L, n=1, batch=1):
    arr = (pi.PiLayer * n)(*([L] * n))
    return pi.lib().pi_workspace_bytes(ctypes.cast(arr, ctypes.c_void_p), n, batch)


def predict(pi, L, x=FAKE, batch=1, idx=FAKE, count=FAKE, ws=FAKE, ws_bytes_=None):
    if ws_bytes_ is None:
        ws_bytes_ = 1 << 30
    return pi.lib().pi_predict(ctypes.byref(L), x, batch, None, None, idx, count, ws, ws_bytes_, None)


def test_workspace_bytes(pi):
    L = make_layer(pi)
    n = ws_bytes(pi, L)
    assert n > 0 and n % 256 == 0
    assert ws_bytes(pi, make_layer(pi, d=100)) == 0
    assert ws_bytes(pi, L, batch=0) == 0 and ws_bytes(pi, L, batch=33) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), 1), (dict(d=100), 1), (dict(rank=48), 1), (dict(ffn=0), 1),
    (dict(act=7), 1), (dict(w_dtype=9), 1), (dict(p_dtype=2), 2), (dict(p_dtype=5), 1),
    (dict(act=1), 1),                                  # ReGLU without a gate matrix
    (dict(A=FAKE + 4), 1), (dict(B=None), 1),          # misaligned / missing predictor
    (dict(pbias=FAKE + 4), 1),
    (dict(w_dtype=2), 1),                              # Q4_0 without scales
    (dict(d=16384 + 64), 2), (dict(rank=4096 + 64), 2),  # beyond the LDS staging limits
    (dict(ffn=(1 << 21) + 1), 2),                      # beyond the score kernel's LDS lists
    (dict(hot=-1), 1), (dict(hot=1001), 1),             # hot prefix outside [0, ffn]
])
def test_predict_rejects_bad_layers(pi, kw, status):
    assert predict(pi, make_layer(pi, **kw)) == status


def test_predict_rejects_bad_arguments(pi):
    L = make_layer(pi)
    assert predict(pi, L, x=None) == 1
    assert predict(pi, L, x=FAKE + 8) == 1
    assert predict(pi, L, idx=None) == 1
    assert predict(pi, L, batch=0) == 1
    assert predict(pi, L, batch=33) == 1
    assert predict(pi, L, ws=None) == 3
    assert predict(pi, L, ws_bytes_=ws_bytes(pi, L) - 1) == 3


def test_q4_layer_with_scales_passes_layer_checks(pi):
    q = pi.PiMat(FAKE, FAKE)
    L = make_layer(pi, w_dtype=pi.PI_Q4_0, up=q, downT=q)
    # accepted by the layer checks; the undersized workspace is what fails
    assert predict(pi, L, ws_bytes_=16) == 3


def test_sparse_ffn_and_stack_validation(pi):
    L = make_layer(pi)
    lib = pi.lib()
    r = lib.pi_sparse_ffn(ctypes.byref(L), FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == 1                                      # batch 1 takes no per-sequence mask
    r = lib.pi_sparse_ffn(ctypes.byref(L), FAKE, 1, None, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert r == 1
    arr = (pi.PiLayer * 2)(L, make_layer(pi, d=1024))
    r = lib.pi_ffn_stack(ctypes.cast(arr, ctypes.c_void_p), 2, FAKE, 1, FAKE, None, None, None, FAKE,
                         1 << 30, None)
    assert r == 1                                      # layers of a stack share d
    r = lib.pi_ffn_stack(ctypes.cast(arr, ctypes.c_void_p), 0, FAKE, 1, FAKE, None, None, None, FAKE,
                         1 << 30, None)
    assert r == 1
    # a trace record's mask must be 16-byte aligned
    one = (pi.PiLayer * 1)(L)
    tr = (pi.PiTrace * 1)()
    tr[0].mask = FAKE + 1
    r = lib.pi_ffn_stack(ctypes.cast(one, ctypes.c_void_p), 1, FAKE, 1, FAKE, None, None,
                         ctypes.cast(tr, ctypes.c_void_p), FAKE, 1 << 30, None)
    assert r == 1


def test_batched_validation(pi):
    L = make_layer(pi)
    lib = pi.lib()
    # batch > 1 needs the per-sequence mask in pi_predict and pi_sparse_ffn
    r = lib.pi_predict(ctypes.byref(L), FAKE, 8, None, None, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == 1
    r = lib.pi_sparse_ffn(ctypes.byref(L), FAKE, 8, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None)
    assert r == 1
    # the batched path needs more workspace than batch 1, and an undersized one is refused
    n1, n8, n32 = ws_bytes(pi, L, batch=1), ws_bytes(pi, L, batch=8), ws_bytes(pi, L, batch=32)
    assert 0 < n1 < n8 < n32
    r = lib.pi_predict(ctypes.byref(L), FAKE, 8, None, FAKE, FAKE, FAKE, FAKE, n8 - 1, None)
    assert r == 3


def test_struct_layouts_match_the_header(pi, tmp_path):
    """ctypes mirrors of pi_mat / pi_layer / pi_trace have the C compiler's sizes and offsets."""
    src = tmp_path / "layout.c"
    fields = {"pi_mat": [f for f, _ in pi.PiMat._fields_], "pi_layer": [f for f, _ in pi.PiLayer._fields_],
              "pi_trace": [f for f, _ in pi.PiTrace._fields_]}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "pi.h"', "int main(void) {"]
    for st, fs in fields.items():
        lines.append(f'  printf("{st} %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'  printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                              text=True).stdout.split("\n") if line)
    for st, cls in (("pi_mat", pi.PiMat), ("pi_layer", pi.PiLayer), ("pi_trace", pi.PiTrace)):
        assert int(out[st]) == ctypes.sizeof(cls), st
        for f in fields[st]:
            assert int(out[f"{st}.{f}"]) == getattr(cls, f).offset, f"{st}.{f}"


def test_static_stack_checks_come_before_any_hip_call(pi):
    """pi_ffn_stack_static refuses bad arguments and a workspace beyond its fixed array
    on the host, so these calls return without touching a GPU."""
    lib = pi.lib()
    L = make_layer(pi)
    one = (pi.PiLayer * 1)(L)
    assert lib.pi_ffn_stack_static(ctypes.cast(one, ctypes.c_void_p), 1, None, 1, FAKE, None, None, None,
                                   None) == 1
    assert lib.pi_ffn_stack_static(ctypes.cast(one, ctypes.c_void_p), 1, FAKE, 33, FAKE, None, None, None,
                                   None) == 1
    q4 = pi.PiMat(FAKE, FAKE)
    big = make_layer(pi, d=16384, rank=4096, ffn=65536, act=pi.PI_REGLU, w_dtype=pi.PI_Q4_0, gate=q4, up=q4,
                     downT=q4)                             # the largest batched shape
    assert ws_bytes(pi, big, batch=32) > pi.STATIC_WORKSPACE_BYTES
    arr = (pi.PiLayer * 1)(big)
    assert lib.pi_ffn_stack_static(ctypes.cast(arr, ctypes.c_void_p), 1, FAKE, 32, FAKE, None, None, None,
                                   None) == 3
    # batch 1 at the largest accepted ffn fits
    assert 0 < ws_bytes(pi, make_layer(pi, d=16384, rank=4096, ffn=1 << 21)) <= pi.STATIC_WORKSPACE_BYTES


@pytest.mark.parametrize("act,wt,fits", [("RELU", "Q4_0", True), ("RELU2", "Q4_0", True), ("RELU", "F32", True),
                                         ("REGLU", "F16", True), ("REGLU", "F32", True), ("REGLU", "Q4_0", False)])
def test_static_workspace_coverage_stated_in_the_header(pi, act, wt, fits):
    """At d = 12288, ffn = 49152, rank = 1024 and batch 2..32 the fixed array holds every
    layer but ReGLU with Q4_0 weights (the K-split up GEMM's partial z for two matrices)."""
    sc = FAKE if wt == "Q4_0" else None
    mats = {k: pi.PiMat(FAKE, sc) for k in ("up", "downT")}
    if act == "REGLU":
        mats["gate"] = pi.PiMat(FAKE, sc)
    L = make_layer(pi, d=12288, ffn=49152, rank=1024, act=getattr(pi, "PI_" + act), w_dtype=getattr(pi, "PI_" + wt),
                   p_dtype=pi.PI_F32 if wt == "F32" else pi.PI_F16, **mats)
    for b in (1, 2, 8, 32):
        n = ws_bytes(pi, L, batch=b)
        assert n > 0
        assert (n <= pi.STATIC_WORKSPACE_BYTES) == (fits or b == 1), (b, n)


def test_static_workspace_size_matches_the_header(pi):
    with open(os.path.join(ROOT, "include", "pi.h")) as fh:
        m = re.search(r"#define PI_STATIC_WORKSPACE_BYTES \((\d+)u << (\d+)\)", fh.read())
    assert pi.STATIC_WORKSPACE_BYTES == int(m.group(1)) << int(m.group(2))
