#!/usr/bin/env python3
"""Decode-time sparse-FFN benchmark on one MI355X.

A step is one decode token (batch 1) through a whole FFN stack: for every
layer the predictor, threshold and compaction, the gathered up/gate GEMV with
its activation, the down projection over the active neurons and the residual
RMS glue -- every step of the hot path, in the library's HIP kernels, behind
the C ABI.  Token t's input is its own seeded x ~ N(0, I); weights are the
seeded synthetic workload (Zipf firing probabilities, hot-first storage) at
the real FFN shapes, generated on the host and resident in HBM before the
timed region starts.

Default workload: the LLaMA(ReLU)-2-7B-shaped ReGLU stack (32 layers, d=4096,
ffn=11008, predictor rank 1024, fp16 weights and predictor, fp32
accumulation), 8 warm-up and 128 timed tokens, token-major (weights are
re-streamed for every token).

Prints one JSON line: tokens/s, the HBM roofline of the dominant kernel on
algorithmic (active) bytes, and the CPU oracle timed on a bounded sample of
the same tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=1, help="workload index (0..4)")
    ap.add_argument("--layers", type=int, default=0, help="override the number of layers (0 = all)")
    ap.add_argument("--order", default="hot_first", choices=["hot_first", "identity"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle budget (a bounded sample of the same tokens); 0 = skip")
    ap.add_argument("--repeats", type=int, default=3, help="timed repeats; the median is reported")
    return ap.parse_args()


def layer_bytes(cfg, k):
    """Algorithmic HBM bytes of one layer for one token at batch 1 with k active neurons.

    Dense predictor (A, B), the predictor bias, the active rows of gate/up and
    down with their bias, the index list, and the x/y vectors.  Rows of
    inactive neurons are not counted.
    """
    pb = {"f32": 4, "f16": 2}[cfg.p_dtype]
    wb = {"f32": 4.0, "f16": 2.0, "q4_0": 18.0 / 32.0}[cfg.w_dtype]
    n_mat = 3 if cfg.act == "reglu" else 2
    d, f, r = cfg.d, cfg.ffn, cfg.rank
    return (r * d + f * r) * pb + 4 * f + k * (n_mat * d * wb + 4) + 4 * k + 8 * d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (asked for {args.gpus}); "
              "the sparse FFN is not sharded across GPUs here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import activation_sparse_predict_amd as pi
    import workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    pi.lib()   # raises if the HIP library is not built

    cfg = workload.CONFIGS[args.config]
    if args.layers:
        cfg = cfg.with_(n_layers=args.layers)
    nthr = min(16, os.cpu_count() or 1)
    W, K = args.warmup, args.steps
    log(f"[bench] {cfg.name}: L={cfg.n_layers} d={cfg.d} f={cfg.ffn} r={cfg.rank} "
        f"{cfg.w_dtype}/{cfg.p_dtype} {cfg.act}; warmup {W}, steps {K}")

    # ---- weights: generated per layer on the host, uploaded, host copy kept
    # only for the layers the CPU oracle will need (all of them, when it runs)
    t0 = time.time()
    keep_host = args.cpu_seconds > 0
    host, layers = [], []
    for l in range(cfg.n_layers):
        lw = workload.make_layer(cfg, l, order=args.order, nthreads=nthr)
        layers.append(pi.DeviceLayer.upload(lw, dev))
        if keep_host:
            host.append(lw)
        del lw
    torch.cuda.synchronize()
    wbytes = sum(L.nbytes() for L in layers)
    log(f"[bench] generated + uploaded {wbytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")

    xs_host = workload.make_tokens(cfg, W + K)[:, 0, :]          # [W+K][d] float32
    xs = torch.from_numpy(np.ascontiguousarray(xs_host)).to(dev)
    outs = torch.empty_like(xs)
    counts = torch.zeros((W + K, cfg.n_layers), dtype=torch.int32, device=dev)

    stream = torch.cuda.Stream()
    stack = pi.Stack(layers)

    # ---- one HIP graph per token slot (x_t -> out_t, counts_t), captured once
    with torch.cuda.stream(stream):
        stack(xs[0], outs[0], counts[0], stream=stream)          # eager warm-up of the path
    stream.synchronize()
    graphs = []
    for t in range(W + K):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            stack(xs[t], outs[t], counts[t], stream=torch.cuda.current_stream())
        graphs.append(g)
    torch.cuda.synchronize()
    log(f"[bench] captured {len(graphs)} token graphs")

    times = []
    for rep in range(args.repeats):
        with torch.cuda.stream(stream):
            for t in range(W):
                graphs[t].replay()
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for t in range(W, W + K):
                graphs[t].replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1)
        times.append(ms)
        log(f"[bench] repeat {rep}: {K} tokens in {ms:.3f} ms ({K / ms * 1e3:.1f} tok/s)")
    ms = float(np.median(times))
    ms_per_step = ms / K

    cnt = counts[W:].cpu().numpy().astype(np.int64)                # [K][L]
    alg_bytes = float(sum(layer_bytes(cfg, int(k)) for k in cnt.ravel())) / K   # per token
    achieved = alg_bytes / (ms_per_step * 1e-3) / 1e9
    mean_active = float(cnt.mean() / cfg.ffn)
    log(f"[bench] mean active {mean_active:.4f}, {alg_bytes / 1e6:.2f} MB/token, "
        f"{achieved:.1f} GB/s ({achieved / HBM_PEAK_GBS:.3f} of peak)")

    # ---- CPU oracle on a bounded sample of the same tokens
    cpu = None
    if keep_host:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = 1
        outs_h = outs.cpu().numpy()
        n_done, errs = 0, []
        tc0 = time.perf_counter()
        for t in range(W, W + K):
            ref = oracle.stack_forward(host, xs_host[t][None, :])
            n_done += 1
            y = ref["out"][0]
            errs.append(float(np.abs(outs_h[t] - y).max() / max(np.abs(y).max(), 1e-30)))
            if time.perf_counter() - tc0 >= args.cpu_seconds:
                break
        tc = time.perf_counter() - tc0
        cpu = {"value": n_done / tc, "unit": "tokens/s", "cores": int(blas_threads),
               "kind": "oracle",
               "sample": f"first {n_done} timed token(s) through all {cfg.n_layers} layers, "
                         f"float64 NumPy oracle, {tc:.1f} s",
               "max_rel_err_vs_gpu_out": max(errs)}
        log(f"[bench] oracle: {n_done} tokens in {tc:.1f} s; max rel err of GPU stack output "
            f"{max(errs):.2e}")

    res = {
        "metric": "sparse-FFN tokens/s at batch 1 (1 GPU)",
        "value": K / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if cfg.w_dtype == "f16" else cfg.w_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "d": cfg.d, "ffn": cfg.ffn,
                   "rank": cfg.rank, "batch": 1, "act": cfg.act, "w_dtype": cfg.w_dtype,
                   "p_dtype": cfg.p_dtype, "order": args.order, "mean_active": mean_active,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "pi_ffn_stack, one token (all kernels of all layers)",
                     "alg_bytes_per_launch": alg_bytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
