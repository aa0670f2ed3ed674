"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

All inputs are seeded and synthetic (workload/).  Small cases span several
tiles and a ragged tail; the full-size cases use the real layer shapes of the
five workloads (fewer layers than the full stacks, same kernels and launch
configuration as the benchmark).
"""
import sys

import numpy as np
import pytest

import oracle
import workload
from parity import BAND, TOL, check_list, check_nz_count, check_scores_masks, check_y, rel_err, replay_stack

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import activation_sparse_predict_amd as pi  # noqa: E402

DEV = "cuda:0"
SENTINEL = -12345.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# Small variants: several tiles plus a ragged ffn tail, every dtype/act pair.
SMALL = {
    "f32-relu": workload.CONFIGS[0].with_(d=512, ffn=2085, rank=64),
    "f16-reglu": workload.CONFIGS[1].with_(d=1024, ffn=3001, rank=128, n_layers=3),
    "f16-relu": workload.CONFIGS[2].with_(d=1024, ffn=4099, rank=256, n_layers=3),
    "q4-relu": workload.CONFIGS[4].with_(d=1024, ffn=3001, rank=128, n_layers=3),
    "q4-reglu": workload.CONFIGS[4].with_(act="reglu", d=512, ffn=1500, rank=64, n_layers=2),
    "f32w-f16p-relu": workload.CONFIGS[0].with_(p_dtype="f16", d=256, ffn=777, rank=64, n_layers=2),
    "f16-relu2": workload.CONFIGS[2].with_(act="relu2", d=512, ffn=2085, rank=128, n_layers=3),
    "q4-relu2": workload.CONFIGS[4].with_(act="relu2", d=512, ffn=1500, rank=64, n_layers=2),
}


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def with_canary(n, dtype, fill=0):
    """A device buffer of n elements followed by 64 canary elements."""
    t = torch.full((n + 64,), fill, dtype=dtype, device=DEV)
    t[n:] = SENTINEL if dtype.is_floating_point else -7
    return t


def canary_ok(t, n):
    tail = t[n:].cpu()
    return bool(torch.all(tail == (SENTINEL if t.dtype.is_floating_point else -7)))


_cache = {}


def host_layers(cfg, n=None):
    key = (cfg, n)
    if key not in _cache:
        _cache.clear()
        n = cfg.n_layers if n is None else n
        _cache[key] = [workload.make_layer(cfg, l) for l in range(n)]
    return _cache[key]


def run_predict(L, x):
    f = L.ffn
    scores = with_canary(f, torch.float32)
    mask = with_canary(f, torch.uint8)
    idx = with_canary(f, torch.int32, -1)
    count = with_canary(1, torch.int32, -1)
    pi.predict(L, dev(x), idx, count, scores=scores, mask=mask)
    torch.cuda.synchronize()
    for t, n in ((scores, f), (mask, f), (idx, f), (count, 1)):
        assert canary_ok(t, n), "write past the end of an output buffer"
    return (scores[:f].cpu().numpy(), mask[:f].cpu().numpy(), idx[:f].cpu().numpy(),
            int(count[0].item()))


def run_sparse_ffn(L, x, idx_list, count=None):
    d = L.d
    n = max(1, len(idx_list))
    idx = torch.zeros(n, dtype=torch.int32, device=DEV)
    if len(idx_list):
        idx[:len(idx_list)] = dev(np.asarray(idx_list, np.int32))
    cnt = torch.tensor([len(idx_list) if count is None else count], dtype=torch.int32, device=DEV)
    y = with_canary(d, torch.float32, float("nan"))
    pi.sparse_ffn(L, dev(x), idx, cnt, y)
    torch.cuda.synchronize()
    assert canary_ok(y, d)
    return y[:d].cpu().numpy()


# -------------------------------------------------------------- predict + ffn
@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    cfg = SMALL[name]
    say(f"[layer_small] {name} d={cfg.d} f={cfg.ffn} r={cfg.rank} {cfg.w_dtype}/{cfg.p_dtype} {cfg.act}")
    lw = workload.make_layer(cfg, 0)
    L = pi.DeviceLayer.upload(lw, DEV)
    for tok in range(3):
        x = workload.make_x(cfg, tok)
        ref = oracle.layer_forward(lw, x)
        scores, mask, idx, count = run_predict(L, x[0])
        st = check_scores_masks(ref["scores"][0], scores, mask)
        check_list(mask, idx, count)
        # FFN over the oracle's own list (so both sides use one set of neurons)
        y = run_sparse_ffn(L, x[0], ref["idx"])
        e = check_y(y, ref["y"][0], TOL[cfg.w_dtype])
        say(f"  tok {tok}: count {count} band {st['band']} flips {st['band_flips']} "
            f"score err {st['max_score_err']:.2e} y err {e:.2e}")


@pytest.mark.parametrize("name", ["f16-reglu", "q4-relu", "f32-relu", "f16-relu2"])
def test_sparse_ffn_edge_cases(name):
    cfg = SMALL[name]
    say(f"[edge] {name}")
    lw = workload.make_layer(cfg, 0)
    L = pi.DeviceLayer.upload(lw, DEV)
    x = workload.make_x(cfg, 5)
    f = cfg.ffn
    args = (cfg.act, lw.gate, lw.up, lw.downT, lw.bias)
    # empty list: y == 0 exactly
    y = run_sparse_ffn(L, x[0], [])
    assert np.array_equal(y, np.zeros_like(y))
    # all neurons: the dense FFN (identity that an all-ones mask gives the dense result)
    y = run_sparse_ffn(L, x[0], np.arange(f))
    check_y(y, oracle.dense_ffn(*args, x)[0], TOL[cfg.w_dtype])
    # count above ffn is clamped to ffn
    y2 = run_sparse_ffn(L, x[0], np.arange(f), count=f + 1000)
    assert np.array_equal(y, y2)
    # unordered list, and entries out of range are skipped
    rng = np.random.default_rng(1)
    sel = np.sort(rng.choice(f, size=f // 7, replace=False))
    ref = oracle.sparse_ffn(*args, x, np.isin(np.arange(f), sel)[None, :])[0]
    check_y(run_sparse_ffn(L, x[0], sel[::-1].copy()), ref, TOL[cfg.w_dtype])
    bad = np.concatenate([sel, [-1, f, f + 5, 2 ** 31 - 1]])
    check_y(run_sparse_ffn(L, x[0], bad), ref, TOL[cfg.w_dtype])


def _poison(lw, keep):
    """Copy of a layer whose rows outside `keep` are NaN in gate/up/downT."""
    import copy
    p = copy.copy(lw)
    drop = np.setdiff1d(np.arange(lw.cfg.ffn), keep)

    def pz(m):
        if m is None:
            return None
        if isinstance(m, workload.Q4Matrix):
            sc = m.scales.copy()
            sc[drop] = np.float16(np.nan).view(np.uint16)
            return workload.Q4Matrix(m.nibbles, sc)
        m2 = m.copy()
        m2[drop] = np.nan
        return m2
    p.gate, p.up, p.downT = pz(lw.gate), pz(lw.up), pz(lw.downT)
    return p


@pytest.mark.parametrize("name", ["f16-reglu", "q4-relu", "f32-relu"])
def test_inactive_rows_are_never_read(name):
    """NaN in every inactive row of gate/up/downT leaves the output unchanged and finite."""
    cfg = SMALL[name].with_(n_layers=1)
    say(f"[poison] {name}")
    lw = workload.make_layer(cfg, 0)
    for tok in range(20):
        x = workload.make_x(cfg, 100 + tok)
        ref = oracle.layer_forward(lw, x)
        if (np.abs(ref["scores"]) < BAND).any():
            continue            # a neuron in the band may legitimately be decided either way
        break
    else:
        pytest.skip("no band-free token found")
    P = pi.DeviceLayer.upload(_poison(lw, ref["idx"]), DEV)
    y = run_sparse_ffn(P, x[0], ref["idx"])
    check_y(y, ref["y"][0], TOL[cfg.w_dtype])
    out = torch.empty(cfg.d, dtype=torch.float32, device=DEV)
    counts = torch.zeros(1, dtype=torch.int32, device=DEV)
    pi.ffn_stack([P], dev(x[0]), out, counts)
    torch.cuda.synchronize()
    assert int(counts[0].item()) == ref["count"]
    o = out.cpu().numpy()
    check_y(o, oracle.rms_glue(x, ref["y"])[0], max(TOL[cfg.w_dtype], 1e-5))


def test_predictor_degenerate_cases():
    cfg = SMALL["f16-relu"].with_(n_layers=1)
    say("[degenerate] zero predictor weights, all-negative and all-positive bias")
    lw = workload.make_layer(cfg, 0)
    import copy
    z = copy.copy(lw)
    z.A = np.zeros_like(lw.A)
    z.B = np.zeros_like(lw.B)
    x = workload.make_x(cfg, 3)
    for sign, expect in ((-1.0, 0), (1.0, cfg.ffn)):
        z.pbias = (sign * (np.abs(lw.bias) + 0.5)).astype(np.float32)
        L = pi.DeviceLayer.upload(z, DEV)
        scores, mask, idx, count = run_predict(L, x[0])
        assert count == expect
        assert np.array_equal(scores, z.pbias)          # s = c exactly when A = B = 0
        check_list(mask, idx, count)
        out = torch.empty(cfg.d, dtype=torch.float32, device=DEV)
        pi.ffn_stack([L], dev(x[0]), out)
        torch.cuda.synchronize()
        ref = oracle.stack_forward([z], x)
        check_y(out.cpu().numpy(), ref["out"][0], TOL[cfg.w_dtype])


# ----------------------------------------------------------------------- stack
def run_stack_traced(layers, x, cfg):
    n, d, f = len(layers), cfg.d, cfg.ffn
    recs = []
    for _ in range(n):
        recs.append(dict(x_in=with_canary(d, torch.float32), scores=with_canary(f, torch.float32),
                         mask=with_canary(f, torch.uint8), idx=with_canary(f, torch.int32, -1),
                         count=with_canary(1, torch.int32, -1), y=with_canary(d, torch.float32)))
    out = with_canary(d, torch.float32)
    counts = with_canary(n, torch.int32, -1)
    nz = with_canary(n, torch.int32, -1)
    trace = pi.make_trace(n, recs)
    pi.ffn_stack(layers, dev(x), out, counts, trace, nz_counts=nz)
    torch.cuda.synchronize()
    assert canary_ok(out, d) and canary_ok(counts, n) and canary_ok(nz, n)
    res = []
    for r in recs:
        sizes = dict(x_in=d, scores=f, mask=f, idx=f, count=1, y=d)
        for k, t in r.items():
            assert canary_ok(t, sizes[k]), k
        res.append(dict(x_in=r["x_in"][:d].cpu().numpy(), scores=r["scores"][:f].cpu().numpy(),
                        mask=r["mask"][:f].cpu().numpy(), idx=r["idx"][:f].cpu().numpy(),
                        count=int(r["count"][0].item()), y=r["y"][:d].cpu().numpy()))
    cts = counts[:n].cpu().numpy()
    assert [r["count"] for r in res] == cts.tolist()
    for r, v in zip(res, nz[:n].cpu().numpy().tolist()):
        assert 0 <= v <= r["count"]
        r["nz"] = v
    return out[:d].cpu().numpy(), res


@pytest.mark.parametrize("name", ["f16-reglu", "f16-relu", "q4-relu", "q4-reglu", "f32w-f16p-relu", "f16-relu2",
                                  "q4-relu2"])
def test_stack_small(name):
    cfg = SMALL[name]
    say(f"[stack_small] {name} L={cfg.n_layers}")
    host = host_layers(cfg)
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    for tok in range(4):
        x = workload.make_x(cfg, 40 + tok)
        out, trace = run_stack_traced(layers, x[0], cfg)
        st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
        say(f"  tok {tok}: {st}; rows read {[t['nz'] for t in trace]} of {[t['count'] for t in trace]}")


def test_stack_deterministic_and_graph_replay():
    cfg = SMALL["f16-reglu"]
    say("[determinism] two eager runs and graph replays are bit-identical")
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host_layers(cfg)]
    stack = pi.Stack(layers)
    x = dev(workload.make_x(cfg, 7)[0])
    outs, cnts = [], []
    for _ in range(2):
        out = torch.empty(cfg.d, dtype=torch.float32, device=DEV)
        counts = torch.zeros(cfg.n_layers, dtype=torch.int32, device=DEV)
        stack(x, out, counts)
        torch.cuda.synchronize()
        outs.append(out.cpu())
        cnts.append(counts.cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(cnts[0], cnts[1])
    # HIP graph: capture once, replay several times with eager work in between
    g_out = torch.empty(cfg.d, dtype=torch.float32, device=DEV)
    g_cnt = torch.zeros(cfg.n_layers, dtype=torch.int32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        stack(x, g_out, g_cnt)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        stack(x, g_out, g_cnt)
    for rep in range(4):
        g_out.fill_(float("nan"))
        g_cnt.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out.cpu(), outs[0]), rep
        assert torch.equal(g_cnt.cpu(), cnts[0]), rep
        _ = (torch.randn(1000, device=DEV) * 2).sum().item()   # unrelated eager work


@pytest.mark.parametrize("nb", [1, 8])
def test_trace_events_in_hip_graph(nb):
    """Timing events of a trace record, eager and as event nodes of a captured graph (the
    benchmark's launch setup): every kernel interval is positive, the output is unchanged."""
    cfg = SMALL["f16-reglu"]
    say(f"[events] batch {nb}: per-kernel events, eager and in a captured graph")
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host_layers(cfg)]
    n, nk = cfg.n_layers, len(pi.LAYER_KERNELS[1 if nb == 1 else 2])
    stack = pi.Stack(layers, batch=nb)
    x = dev(workload.make_x(cfg, 5, seqs=nb))
    ref = torch.empty(nb, cfg.d, device=DEV)
    stack(x, ref)
    torch.cuda.synchronize()
    evs = [[pi.HipEvent() for _ in range(nk + 1)] for _ in range(n)]
    trace = pi.make_trace(n, [{"events": [int(e) for e in ev]} for ev in evs])
    s = torch.cuda.Stream()
    out = torch.full((nb, cfg.d), float("nan"), device=DEV)
    torch.cuda.synchronize()
    stack(x, out, None, trace, stream=s)
    s.synchronize()
    assert torch.equal(out.cpu(), ref.cpu())
    eager = [[ev[i].elapsed_ms(ev[i + 1]) for i in range(nk)] for ev in evs]
    assert all(v > 0 for row in eager for v in row), eager
    graph = pi.HipGraph(s, lambda st: stack(x, out, None, trace, stream=st))
    for rep in range(3):
        for ev in evs:                  # stamp in reverse order: every interval <= 0 until replayed
            for e in reversed(ev):
                e.record(s)
        s.synchronize()
        assert all(ev[i].elapsed_ms(ev[i + 1]) <= 0 for ev in evs for i in range(nk))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        s.synchronize()
        assert torch.equal(out.cpu(), ref.cpu()), rep
        replayed = [[ev[i].elapsed_ms(ev[i + 1]) for i in range(nk)] for ev in evs]
        assert all(v > 0 for row in replayed for v in row), replayed
    say(f"  layer 0 kernel intervals (ms), graph: {[round(v, 4) for v in replayed[0]]}")


# ------------------------------------------------------------------ full size
# (workload, layers, tokens): the real layer shapes, four layers deep
FULL_CASES = [(0, 1, 16), (1, 4, 3), (2, 4, 2), (3, 4, 2), (4, 4, 2)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("ci,n_layers,n_tok", FULL_CASES, ids=lambda v: str(v))
def test_full_size_stack(ci, n_layers, n_tok):
    """Real layer shapes (d, ffn, rank, dtype) of each workload, in the benchmark's launch
    setup, every layer replayed layer-locally."""
    cfg = workload.CONFIGS[ci]
    say(f"[full] config {ci} {cfg.name}: {n_layers} layers, {n_tok} tokens")
    host = [workload.make_layer(cfg, l, nthreads=16) for l in range(n_layers)]
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    worst_y, worst_e2e, flips = 0.0, 0.0, 0
    for tok in range(n_tok):
        x = workload.make_x(cfg, tok)
        out, trace = run_stack_traced(layers, x[0], cfg)
        st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
        worst_y = max(worst_y, st["max_y_err"])
        worst_e2e = max(worst_e2e, st["out_err_end_to_end"])
        flips += st["band_flips"]
        rate = np.mean([t["count"] / cfg.ffn for t in trace])
        nzr = np.mean([t["nz"] / max(t["count"], 1) for t in trace])
        say(f"  tok {tok}: active {rate:.3f} (h != 0: {nzr:.3f} of them) band {st['band']} "
            f"flips {st['band_flips']} score err {st['max_score_err']:.2e} y err {st['max_y_err']:.2e} "
            f"glue err {st['max_glue_err']:.2e} end-to-end {st['out_err_end_to_end']:.2e}")
    say(f"  worst y err {worst_y:.2e}, worst end-to-end {worst_e2e:.2e}, band flips {flips}")
    if cfg.n_layers == 1:
        # a one-layer stack has no trajectory to diverge: its output is gated end to end
        assert worst_e2e <= max(TOL[cfg.w_dtype], 1e-5)
    del layers
    torch.cuda.empty_cache()


# ------------------------------------------------------------- maximum sizes
# The largest width and rank the library accepts (d <= 16384, rank <= 4096:
# vectors are staged whole in LDS), with a ragged ffn; and the kernel variants
# that only wide rows select: Q4_0 ReGLU with d > 2048 (six chunks per lane
# per gathered row, rows taken in pairs) and fp32 weights with d > 512.
MAX = {
    "f16-reglu": workload.CONFIGS[1].with_(d=16384, ffn=1100, rank=4096, n_layers=2),
    "q4-relu": workload.CONFIGS[4].with_(d=16384, ffn=777, rank=4096, n_layers=2),
    "q4-reglu-d12288": workload.CONFIGS[4].with_(act="reglu", d=12288, ffn=3001, rank=1024, n_layers=3),
    "q4-relu2-d12288": workload.CONFIGS[4].with_(act="relu2", d=12288, ffn=3001, rank=1024, n_layers=3),
    "f32-relu-d4096": workload.CONFIGS[0].with_(d=4096, ffn=5003, rank=256, n_layers=3),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(MAX))
def test_maximum_width_and_rank(name):
    cfg = MAX[name]
    say(f"[max] {name} d={cfg.d} f={cfg.ffn} r={cfg.rank} {cfg.w_dtype}/{cfg.p_dtype} {cfg.act}")
    host = [workload.make_layer(cfg, l, nthreads=16) for l in range(cfg.n_layers)]
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    x = workload.make_x(cfg, 5)
    # single layer: predictor and the FFN over the oracle's list
    ref = oracle.layer_forward(host[0], x)
    scores, mask, idx, count = run_predict(layers[0], x[0])
    check_scores_masks(ref["scores"][0], scores, mask)
    check_list(mask, idx, count)
    check_y(run_sparse_ffn(layers[0], x[0], ref["idx"]), ref["y"][0], TOL[cfg.w_dtype])
    # the stack, every layer replayed layer-locally
    out, trace = run_stack_traced(layers, x[0], cfg)
    st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
    say(f"  count {count}, stack {st}")
    del layers
    torch.cuda.empty_cache()


# ------------------------------------------------------------ hot-dense prefix
@pytest.mark.parametrize("name,hot", [("q4-relu", 300), ("f16-reglu", 257), ("f16-relu2", 1)])
def test_stack_hot_prefix(name, hot):
    """Slots [0, hot) are on without a prediction in every layer: their mask bytes are
    1, their scores are left untouched (the buffers start at 0), and each layer's y
    is the oracle's on the GPU's own input and mask (which now includes the hot prefix)."""
    cfg = SMALL[name]
    say(f"[hot] {name} hot {hot}")
    host = host_layers(cfg)
    for h in host:
        h.hot = hot
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    x = workload.make_x(cfg, 21)
    out, trace = run_stack_traced(layers, x[0], cfg)
    for t in trace:
        assert np.all(t["mask"][:hot] == 1) and t["count"] >= hot
        assert np.array_equal(t["idx"][:hot], np.arange(hot))
        assert np.all(t["scores"][:hot] == 0)                     # untouched: left as the buffer's fill
    st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
    say(f"  {st}")
    # single-layer predictor: the same prefix, and the tail's scores
    L = layers[0]
    scores, mask, idx, count = run_predict(L, x[0])
    assert np.all(mask[:hot] == 1) and np.all(scores[:hot] == 0)
    ref = oracle.layer_forward(host[0], x)
    check_scores_masks(ref["scores"][0][hot:], scores[hot:], mask[hot:])
    check_list(mask.astype(bool), idx, count)


def test_stack_long_score_lists():
    """Every neuron on (hot prefix over the whole ffn, biases that keep every h
    nonzero) at a shape whose score-block lists (64 entries each) are longer than
    what the down projection reads ahead with the counts (32 per list): the
    lists are read again after the counts, and each layer's y is still the
    oracle's on the GPU's own input and mask."""
    cfg = workload.CONFIGS[2].with_(d=512, ffn=32768, rank=64, n_layers=2)
    say(f"[long_lists] d {cfg.d} ffn {cfg.ffn}")
    host = [workload.make_layer(cfg, l) for l in range(cfg.n_layers)]
    for h in host:
        h.hot = cfg.ffn
        h.bias = np.full_like(h.bias, 4.0)
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    x = workload.make_x(cfg, 5)
    out, trace = run_stack_traced(layers, x[0], cfg)
    for t in trace:
        assert t["count"] == cfg.ffn
    st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
    say(f"  {st}")
    del layers
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_full_size_stack_hot_prefix():
    """The OPT-175B-shaped Q4_0 stack with the byte model's hot prefix (hot_count)."""
    cfg = workload.CONFIGS[4]
    n_layers = 2
    host = [workload.make_layer(cfg, l, nthreads=16) for l in range(n_layers)]
    for h in host:
        h.hot = workload.hot_count(cfg, h.p_storage)
    say(f"[full_hot] config 4: {n_layers} layers, hot {[h.hot for h in host]}")
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    x = workload.make_x(cfg, 3)
    out, trace = run_stack_traced(layers, x[0], cfg)
    st = replay_stack(host, trace, out, x, cfg.w_dtype, cfg.act)
    say(f"  counts {[t['count'] for t in trace]}; {st}")
    del layers
    torch.cuda.empty_cache()

