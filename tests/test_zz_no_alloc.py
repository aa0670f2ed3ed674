"""pi_ffn_stack_static (the stack without a workspace argument) against pi_ffn_stack.

Two calls in a row through the C ABI, the second with a smaller input (fewer
layers, a narrower width, a smaller batch), each compared with pi_ffn_stack
on a workspace of its own: the same kernels on the same inputs give the same
bits, so outputs, per-layer counts and rows read must be identical.  The
first call's contents stay in the shared array; the second must not depend
on them.
"""
import sys

import numpy as np
import pytest

import workload

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import activation_sparse_predict_amd as pi  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_both(cfg, nb, tok):
    host = [workload.make_layer(cfg, l) for l in range(cfg.n_layers)]
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    assert pi.workspace_bytes(layers, nb) <= pi.STATIC_WORKSPACE_BYTES
    x = torch.from_numpy(workload.make_x(cfg, tok, seqs=nb)).to(DEV)
    n = cfg.n_layers
    res = []
    for fn in ("static", "workspace"):
        out = torch.full((nb, cfg.d), float("nan"), device=DEV)
        counts = torch.full((n,), -1, dtype=torch.int32, device=DEV)
        nz = torch.full((n,), -1, dtype=torch.int32, device=DEV)
        if fn == "static":
            pi.ffn_stack_static(layers, x, out, counts, batch=nb, nz_counts=nz)
        else:
            pi.ffn_stack(layers, x, out, counts, batch=nb, nz_counts=nz)
        torch.cuda.synchronize()
        res.append((out.cpu(), counts.cpu(), nz.cpu()))
    (o1, c1, z1), (o2, c2, z2) = res
    assert torch.all(torch.isfinite(o1))
    assert torch.equal(o1, o2), float((o1 - o2).abs().max())
    assert torch.equal(c1, c2) and torch.equal(z1, z2)
    return c1.tolist()


@pytest.mark.parametrize("first,second", [
    ((workload.CONFIGS[1].with_(d=1024, ffn=3001, rank=128, n_layers=3), 8),
     (workload.CONFIGS[2].with_(d=512, ffn=1500, rank=64, n_layers=2), 1)),
    ((workload.CONFIGS[4].with_(d=2048, ffn=4099, rank=256, n_layers=3), 1),
     (workload.CONFIGS[4].with_(d=1024, ffn=2085, rank=128, n_layers=2), 1)),
    ((workload.CONFIGS[3].with_(d=1024, ffn=2085, rank=128, n_layers=2), 32),
     (workload.CONFIGS[3].with_(d=512, ffn=1100, rank=64, n_layers=2), 4)),
])
def test_static_entry_point_matches_the_workspace_one(first, second):
    for i, (cfg, nb) in enumerate((first, second)):
        say(f"[no_alloc] call {i + 1}: d={cfg.d} f={cfg.ffn} r={cfg.rank} L={cfg.n_layers} "
            f"{cfg.w_dtype} {cfg.act} batch {nb}")
        counts = run_both(cfg, nb, 20 + i)
        say(f"  counts {counts}: identical to pi_ffn_stack")


def test_static_entry_point_in_a_captured_graph():
    """The entry point is for code under graph capture: capture it, replay it several
    times with eager work in between, and compare every replay with the eager result."""
    cfg = workload.CONFIGS[1].with_(d=1024, ffn=3001, rank=128, n_layers=2)
    layers = [pi.DeviceLayer.upload(workload.make_layer(cfg, l), DEV) for l in range(cfg.n_layers)]
    x = torch.from_numpy(workload.make_x(cfg, 3)).to(DEV)
    ref = torch.empty(1, cfg.d, device=DEV)
    pi.ffn_stack(layers, x, ref)
    torch.cuda.synchronize()
    out = torch.full_like(ref, float("nan"))
    s = pi.HipStream()
    pi.ffn_stack_static(layers, x, out, stream=s)      # first call on this device: symbol lookup
    s.synchronize()
    assert torch.equal(out.cpu(), ref.cpu())
    graph = pi.HipGraph(s, lambda st: pi.ffn_stack_static(layers, x, out, stream=st))
    for rep in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        s.synchronize()
        assert torch.equal(out.cpu(), ref.cpu()), rep
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()
