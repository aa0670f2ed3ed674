"""GPU parity of the batched path (1 < batch <= 32) against the CPU oracle.

Per sequence: scores within the threshold band, masks bit-exact outside it,
the union list equal to the ascending list of the GPU's own union, and each
sequence's FFN output equal to its own single-sequence result (the oracle's
batch semantics).  Single layers are checked on the oracle's masks; stacks by
layer-local replay on the GPU's own inputs and masks, so that a band neuron
decided differently cannot leak into the comparison.
"""
import sys

import numpy as np
import pytest

import oracle
import workload
from parity import BAND, TOL, check_list, check_scores_masks, check_y, rel_err, replay_stack

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import activation_sparse_predict_amd as pi  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


SMALL = {
    "f16-relu": workload.CONFIGS[3].with_(d=1024, ffn=2085, rank=256, n_layers=2),
    "f16-reglu": workload.CONFIGS[1].with_(d=512, ffn=1500, rank=128, n_layers=2),
    "q4-relu": workload.CONFIGS[4].with_(d=1024, ffn=3001, rank=128, n_layers=2),
    "q4-reglu": workload.CONFIGS[4].with_(act="reglu", d=512, ffn=777, rank=64, n_layers=2),
    "f32-relu": workload.CONFIGS[0].with_(d=256, ffn=1000, rank=64, n_layers=2),
    "f16-relu2": workload.CONFIGS[3].with_(act="relu2", d=512, ffn=1500, rank=128, n_layers=2),
}


def run_predict(L, X):
    nb, f = X.shape[0], L.ffn
    scores = torch.full((nb, f), float("nan"), dtype=torch.float32, device=DEV)
    mask = torch.full((nb, f), 7, dtype=torch.uint8, device=DEV)
    idx = torch.full((f,), -1, dtype=torch.int32, device=DEV)
    count = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    pi.predict(L, dev(X), idx, count, scores=scores, mask=mask, batch=nb)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), mask.cpu().numpy(), idx.cpu().numpy(), int(count[0].item())


def run_sparse_ffn(L, X, idx_list, masks):
    nb, d = X.shape
    n = max(1, len(idx_list))
    idx = torch.zeros(n, dtype=torch.int32, device=DEV)
    if len(idx_list):
        idx[:len(idx_list)] = dev(np.asarray(idx_list, np.int32))
    cnt = torch.tensor([len(idx_list)], dtype=torch.int32, device=DEV)
    y = torch.full((nb, d), float("nan"), dtype=torch.float32, device=DEV)
    pi.sparse_ffn(L, dev(X), idx, cnt, y, mask=dev(np.asarray(masks, np.uint8)), batch=nb)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("nb", [2, 8, 32])
@pytest.mark.parametrize("name", list(SMALL))
def test_batch_layer_small(name, nb):
    cfg = SMALL[name]
    say(f"[batch_small] {name} batch {nb} d={cfg.d} f={cfg.ffn} r={cfg.rank}")
    lw = workload.make_layer(cfg, 0)
    L = pi.DeviceLayer.upload(lw, DEV)
    X = workload.make_x(cfg, 3, seqs=nb)
    ref = oracle.layer_forward(lw, X)
    scores, mask, idx, count = run_predict(L, X)
    flips = 0
    for b in range(nb):
        st = check_scores_masks(ref["scores"][b], scores[b], mask[b])
        flips += st["band_flips"]
    union = mask.astype(bool).any(axis=0)
    check_list(union, idx, count)
    # the FFN on the oracle's own masks and union list, per sequence
    Y = run_sparse_ffn(L, X, ref["idx"], ref["masks"])
    for b in range(nb):
        check_y(Y[b], ref["y"][b], TOL[cfg.w_dtype])
    # each sequence equals its own single-sequence result
    single = oracle.layer_forward(lw, X[1:2])
    check_y(Y[1], single["y"][0], TOL[cfg.w_dtype])
    say(f"  union {count} band flips {flips} worst y err "
        f"{max(rel_err(Y[b], ref['y'][b]) for b in range(nb)):.2e}")


def test_batch_edge_cases():
    cfg = SMALL["f16-relu"]
    say("[batch_edge] empty list, all neurons, padded rows")
    lw = workload.make_layer(cfg, 0)
    L = pi.DeviceLayer.upload(lw, DEV)
    nb, f = 5, cfg.ffn
    X = workload.make_x(cfg, 9, seqs=nb)
    Y = run_sparse_ffn(L, X, [], np.zeros((nb, f), bool))
    assert np.array_equal(Y, np.zeros_like(Y))
    ones = np.ones((nb, f), bool)
    Y = run_sparse_ffn(L, X, np.arange(f), ones)
    dense = oracle.dense_ffn(cfg.act, lw.gate, lw.up, lw.downT, lw.bias, X)
    for b in range(nb):
        check_y(Y[b], dense[b], TOL[cfg.w_dtype])
    # a neuron listed for the union but off in a sequence's own mask contributes 0 there
    rng = np.random.default_rng(4)
    M = rng.random((nb, f)) < 0.3
    M[2] = False                                   # sequence 2 has no active neuron at all
    listed = np.flatnonzero(M.any(axis=0))
    Y = run_sparse_ffn(L, X, listed[::-1].copy(), M)   # unordered list
    ref = oracle.sparse_ffn(cfg.act, lw.gate, lw.up, lw.downT, lw.bias, X, M)
    assert np.array_equal(Y[2], np.zeros_like(Y[2]))
    for b in range(nb):
        check_y(Y[b], ref[b], TOL[cfg.w_dtype])


def traced_records(n, nb, d, f):
    return [dict(x_in=torch.empty(nb, d, device=DEV), scores=torch.empty(nb, f, device=DEV),
                 mask=torch.empty(nb, f, dtype=torch.uint8, device=DEV),
                 idx=torch.empty(f, dtype=torch.int32, device=DEV),
                 count=torch.empty(1, dtype=torch.int32, device=DEV),
                 y=torch.full((nb, d), float("nan"), device=DEV)) for _ in range(n)]


def to_host(recs):
    out = []
    for r in recs:
        h = {k: v.cpu().numpy() for k, v in r.items()}
        h["count"] = int(h["count"][0])
        out.append(h)
    return out


def test_batch_stack_deterministic_and_traced():
    cfg = SMALL["f16-reglu"].with_(n_layers=3)
    nb = 8
    say(f"[batch_stack] {cfg.n_layers} layers, batch {nb}, traced")
    host = [workload.make_layer(cfg, l) for l in range(cfg.n_layers)]
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    X = workload.make_x(cfg, 11, seqs=nb)
    d, f, n = cfg.d, cfg.ffn, cfg.n_layers
    stack = pi.Stack(layers, batch=nb)
    outs = []
    for rep in range(2):
        recs = traced_records(n, nb, d, f)
        out = torch.empty(nb, d, device=DEV)
        counts = torch.zeros(n, dtype=torch.int32, device=DEV)
        stack(dev(X), out, counts, pi.make_trace(n, recs))
        torch.cuda.synchronize()
        outs.append((out.cpu(), counts.cpu(), to_host(recs)))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    out, counts, recs = outs[0][0].numpy(), outs[0][1].numpy(), outs[0][2]
    assert [r["count"] for r in recs] == counts.tolist()
    st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act)
    say(f"  {st}")


# (workload, batch, layers, sequences replayed: None = all)
FULL = [(3, 8, 2, None), (3, 32, 2, None), (4, 32, 2, [0, 1, 16, 31])]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci,nb,n_layers,seqs", FULL, ids=lambda v: str(v))
def test_batch_full_size(ci, nb, n_layers, seqs):
    """Real layer shapes of the batched workloads, through the stack, layer-locally replayed."""
    cfg = workload.CONFIGS[ci]
    say(f"[batch_full] config {ci} {cfg.name}: batch {nb}, {n_layers} layers, "
        f"sequences replayed: {'all' if seqs is None else seqs}")
    host = [workload.make_layer(cfg, l, nthreads=16) for l in range(n_layers)]
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    X = workload.make_x(cfg, 0, seqs=nb)
    d, f = cfg.d, cfg.ffn
    recs = traced_records(n_layers, nb, d, f)
    out = torch.empty(nb, d, device=DEV)
    pi.ffn_stack(layers, dev(X), out, trace=pi.make_trace(n_layers, recs), batch=nb)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    recs = to_host(recs)
    del layers
    torch.cuda.empty_cache()
    st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act, seqs=seqs, end_to_end=False)
    say(f"  unions {[r['count'] for r in recs]} of {f}; {st}")


# ------------------------------------------------------------- maximum sizes
def test_batch_maximum_width_and_rank():
    """Batch 32 at the largest width and rank the library accepts (d = 16384, rank = 4096)."""
    cfg = workload.CONFIGS[3].with_(d=16384, ffn=1100, rank=4096, n_layers=1)
    nb = 32
    say(f"[batch_max] d={cfg.d} f={cfg.ffn} r={cfg.rank} batch {nb}")
    lw = workload.make_layer(cfg, 0)
    L = pi.DeviceLayer.upload(lw, DEV)
    X = workload.make_x(cfg, 4, seqs=nb)
    ref = oracle.layer_forward(lw, X)
    scores, mask, idx, count = run_predict(L, X)
    for b in range(nb):
        check_scores_masks(ref["scores"][b], scores[b], mask[b])
    check_list(mask.astype(bool).any(axis=0), idx, count)
    Y = run_sparse_ffn(L, X, ref["idx"], ref["masks"])
    for b in range(nb):
        check_y(Y[b], ref["y"][b], TOL[cfg.w_dtype])
    say(f"  union {count}")


def test_batch_maximum_ffn_every_neuron_active():
    """The largest ffn of the batched path (65536) with every neuron active in every
    sequence: the union list fills each split of the down GEMM to its LDS capacity."""
    cfg = workload.CONFIGS[3].with_(d=64, ffn=65536, rank=64, n_layers=1)
    nb = 8
    lw = workload.make_layer(cfg, 0)
    lw.pbias = np.full(cfg.ffn, 1000.0, np.float32)          # every score far above 0
    say(f"[batch_max_ffn] d={cfg.d} f={cfg.ffn} r={cfg.rank} batch {nb}, all active")
    L = pi.DeviceLayer.upload(lw, DEV)
    X = workload.make_x(cfg, 6, seqs=nb)
    ref = oracle.layer_forward(lw, X)
    assert ref["count"] == cfg.ffn
    scores, mask, idx, count = run_predict(L, X)
    assert count == cfg.ffn and mask.all()
    check_list(mask.astype(bool).any(axis=0), idx, count)
    Y = run_sparse_ffn(L, X, ref["idx"], ref["masks"])
    for b in range(nb):
        check_y(Y[b], ref["y"][b], TOL[cfg.w_dtype])
    # the stack path on the same layer: its union count is every neuron too
    out = torch.empty(nb, cfg.d, device=DEV)
    counts = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    pi.ffn_stack([L], dev(X), out, counts, batch=nb)
    torch.cuda.synchronize()
    assert int(counts[0]) == cfg.ffn
    x_next = oracle.rms_glue(X, ref["y"])
    for b in range(nb):
        check_y(out[b].cpu().numpy(), x_next[b], max(TOL[cfg.w_dtype], 1e-5))



# ------------------------------------------------- activation range (fp16 split)
def _scale_q4(m, factor):
    """A Q4_0 matrix with every block scale multiplied by a power of two (exact in fp16)."""
    s = m.scales.view(np.float16).astype(np.float32) * np.float32(factor)
    return workload.Q4Matrix(m.nibbles, s.astype(np.float16).view(np.uint16))


def test_batch_squared_relu_outputs_beyond_fp16_range():
    """Q4_0 Squared ReLU at d = 12288 whose h exceeds the fp16 range (|h| > 65504):
    the batched FFN splits each row of h into fp16 hi/lo after scaling it by a power
    of two, so the stack still matches the oracle layer by layer."""
    cfg = workload.CONFIGS[4].with_(act="relu2", d=12288, ffn=3001, rank=1024, n_layers=2)
    nb = 8
    say(f"[batch_h_range] q4 relu2 d={cfg.d} f={cfg.ffn} r={cfg.rank} batch {nb}, up scales x 64")
    host = []
    for l in range(cfg.n_layers):
        lw = workload.make_layer(cfg, l, nthreads=16)
        lw.up = _scale_q4(lw.up, 64.0)
        host.append(lw)
    X = workload.make_x(cfg, 2, seqs=nb)
    # the first layer's h, from the oracle's own steps: its largest value is past fp16
    ref = oracle.layer_forward(host[0], X)
    act_rows = ref["idx"]
    Z = oracle.decode_rows(host[0].up, act_rows) @ X.astype(np.float64).T + \
        oracle.ffn_bias(host[0])[act_rows].astype(np.float64)[:, None]
    hmax = float(np.max(np.maximum(Z, 0.0) ** 2 * ref["masks"][:, act_rows].T))
    say(f"  layer 0: max h = {hmax:.3g}")
    assert hmax > 65504.0
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    recs = traced_records(cfg.n_layers, nb, cfg.d, cfg.ffn)
    out = torch.empty(nb, cfg.d, device=DEV)
    pi.ffn_stack(layers, dev(X), out, trace=pi.make_trace(cfg.n_layers, recs), batch=nb)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    recs = to_host(recs)
    assert np.all(np.isfinite(out))
    st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act)
    say(f"  {st}")


@pytest.mark.parametrize("factor", [1e6, 1e-12])
def test_batch_caller_input_of_any_magnitude(factor):
    """The stack's input enters the first layer without a glue: rows far above the fp16
    range, or far below its normal range, are scaled by a power of two before their
    fp16 split, so the first layer's scores and the whole stack stay in parity."""
    cfg = SMALL["f16-relu"].with_(n_layers=2)
    nb = 4
    say(f"[batch_x_range] input x {factor:g}")
    host = [workload.make_layer(cfg, l) for l in range(cfg.n_layers)]
    # the first layer's scores scale with its input: scale its predictor bias with them
    host[0].pbias = (oracle.predictor_bias(host[0]) * np.float32(factor)).astype(np.float32)
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    X = (workload.make_x(cfg, 5, seqs=nb) * np.float32(factor)).astype(np.float32)
    recs = traced_records(cfg.n_layers, nb, cfg.d, cfg.ffn)
    out = torch.empty(nb, cfg.d, device=DEV)
    pi.ffn_stack(layers, dev(X), out, trace=pi.make_trace(cfg.n_layers, recs), batch=nb)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    recs = to_host(recs)
    assert np.all(np.isfinite(out))
    st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act, score_units=[factor, 1.0])
    say(f"  {st}")


def test_batch_hot_prefix():
    """Batched path with a hot-dense prefix: the prefix is on for every sequence (and
    in the union), no prefix score is written, and the stack replays layer by layer."""
    cfg = SMALL["q4-relu"].with_(n_layers=2)
    nb, hot = 8, 77                      # a tile of 32 wholly hot, and one partly
    say(f"[batch_hot] q4 relu batch {nb} hot {hot}")
    host = [workload.make_layer(cfg, l) for l in range(cfg.n_layers)]
    for h in host:
        h.hot = hot
    layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
    X = workload.make_x(cfg, 13, seqs=nb)
    recs = traced_records(cfg.n_layers, nb, cfg.d, cfg.ffn)
    for r in recs:
        r["scores"].fill_(float("nan"))
    out = torch.empty(nb, cfg.d, device=DEV)
    pi.ffn_stack(layers, dev(X), out, trace=pi.make_trace(cfg.n_layers, recs), batch=nb)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    recs = to_host(recs)
    for r in recs:
        assert np.all(r["mask"][:, :hot] == 1) and not np.isfinite(r["scores"][:, :hot]).any()
    st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act)
    say(f"  {st}")
    # the batched predictor on its own
    scores, mask, idx, count = run_predict(layers[0], X)
    ref = oracle.layer_forward(host[0], X)
    assert np.all(mask[:, :hot] == 1) and not np.isfinite(scores[:, :hot]).any()
    for b in range(nb):
        check_scores_masks(ref["scores"][b][hot:], scores[b][hot:], mask[b][hot:])
    check_list(mask.astype(bool).any(axis=0), idx, count)



# ------------------------- chunk counts of the pipelined down projections
# The Q4_0 and fp16 down projections take their split of the union in chunks of 128
# positions, in a loop of four steps and then 1..3 straight-line steps.  At d = 1024
# there are 16 splits, so a union of 128 * 16 * k rows gives every split k chunks;
# d = 4160 has 17 column groups (a block count that is no multiple of 8, and column
# tiles past d in the last group).
REMAINDER_CASES = [(1024, 128 * 16 * 2), (1024, 128 * 16 * 3), (1024, 128 * 16 * 5 - 77),
                   (1024, 128 * 16 * 8), (4160, 1500)]


@pytest.mark.parametrize("name", ["q4-relu", "f16-relu"])
def test_batch_down_chunk_remainders(name):
    """pi_sparse_ffn over explicit unions whose splits hold 2, 3, 5 (the last chunk
    ragged) and 8 chunks, gathered and dense, against the oracle; every sequence's
    mask a random half of the union."""
    nb = 8
    rng = np.random.default_rng(2024)
    for d, n in REMAINDER_CASES:
        cfg = SMALL[name].with_(d=d, ffn=max(16384 + 111, n + 111) if d == 1024 else 3001, n_layers=1)
        say(f"[batch_chunks] {name} d={d} f={cfg.ffn} union {n} batch {nb}")
        lw = workload.make_layer(cfg, 0)
        X = workload.make_x(cfg, 5, seqs=nb)
        union = np.sort(rng.choice(cfg.ffn, size=n, replace=False)).astype(np.int32)
        M = np.zeros((nb, cfg.ffn), np.uint8)
        for b in range(nb):
            M[b, union[rng.random(n) < 0.5]] = 1
        Yr = oracle.sparse_ffn(cfg.act, lw.gate, lw.up, lw.downT, oracle.ffn_bias(lw), X, M)
        for tag, frac in (("gathered", 2.0), ("dense", 1e-6)) if d == 1024 else (("gathered", 2.0),):
            lw.dense_frac = frac
            L = pi.DeviceLayer.upload(lw, DEV)
            Y = run_sparse_ffn(L, X, union, M)
            for b in range(nb):
                check_y(Y[b], Yr[b], TOL[cfg.w_dtype])
            say(f"  {tag}: max rel err {max(rel_err(Y[b], Yr[b]) for b in range(nb)):.2e}")
            del L


# ------------------------------------------- dense fallback at a large union
def _high_union_layer(cfg, layer, shift):
    lw = workload.make_layer(cfg, layer)
    lw.pbias = (oracle.predictor_bias(lw) + np.float32(shift)).astype(np.float32)
    return lw


@pytest.mark.parametrize("name", ["f16-relu", "q4-reglu", "f32-relu"])
def test_batch_dense_fallback(name):
    """Above the union threshold the batched FFN runs over every neuron in storage order
    (neurons outside the union get h = 0): forced on (dense_frac tiny) and off (above 1),
    both agree with the oracle, through the stack and through pi_sparse_ffn with an
    explicit list (whose other neurons' mask bytes must read as 0)."""
    cfg = SMALL[name].with_(n_layers=2)
    nb = 8
    say(f"[batch_dense] {name} batch {nb}")
    host = [_high_union_layer(cfg, l, 1.0) for l in range(cfg.n_layers)]
    X = workload.make_x(cfg, 17, seqs=nb)
    ref0 = oracle.layer_forward(host[0], X)
    say(f"  layer 0 union {ref0['count']} of {cfg.ffn}")
    for tag, frac in (("dense", 1e-6), ("gathered", 2.0)):
        for h in host:
            h.dense_frac = frac
        layers = [pi.DeviceLayer.upload(h, DEV) for h in host]
        recs = traced_records(cfg.n_layers, nb, cfg.d, cfg.ffn)
        out = torch.empty(nb, cfg.d, device=DEV)
        pi.ffn_stack(layers, dev(X), out, trace=pi.make_trace(cfg.n_layers, recs), batch=nb)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        recs = to_host(recs)
        st = replay_stack(host, recs, out, X, cfg.w_dtype, cfg.act)
        say(f"  {tag}: {st}")
        # explicit list: a third of the union, in its own order, with per-sequence masks
        M = ref0["masks"].copy()
        keep = ref0["idx"][::3]
        Mk = np.zeros_like(M)
        Mk[:, keep] = M[:, keep]
        Y = run_sparse_ffn(layers[0], X, keep[::-1].copy(), Mk)
        Yr = oracle.sparse_ffn(cfg.act, host[0].gate, host[0].up, host[0].downT, oracle.ffn_bias(host[0]), X, Mk)
        for b in range(nb):
            check_y(Y[b], Yr[b], TOL[cfg.w_dtype])
