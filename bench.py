#!/usr/bin/env python3
"""Decode-time sparse-FFN benchmark on one MI355X.

A step is one decode token through a whole FFN stack (batch 1), or one decode
step of B independent sequences (--batch B): for every layer the predictor,
threshold and compaction, the gathered up/gate projection with its
activation, the down projection over the active neurons and the residual RMS
glue -- every step of the hot path, in the library's HIP kernels, behind the
C ABI.  Token t's input is its own seeded x ~ N(0, I) per sequence; weights
are the seeded synthetic workload (Zipf firing probabilities, hot-first
storage) at the real FFN shapes, generated on the host one layer at a time
and resident in HBM before the timed region starts.

Default workload: the OPT-175B-shaped ReLU stack with Q4_0 weights (96
layers, d=12288, ffn=49152, fp16 predictor of rank 1024, fp32 accumulation),
batch 1, 8 warm-up and 128 timed tokens, token-major (weights are re-streamed
for every token).

Timing: one HIP graph per token slot, replayed on one stream, bracketed by
events; the median of the repeats is reported.  In every fourth token graph
the kernels of one layer (rotating over the layers) are bracketed by event
nodes, so per-kernel durations are sampled live over the timed region on the
stream the kernels run on.  An event node adds a fixed cost to each interval;
it is measured in the same run by pairing each such slot with one that
brackets only the whole layer, and subtracted.

CPU baseline: the float64 oracle runs layer-major while the layers are
generated (each host layer is dropped after its upload), on the first timed
token(s), until its time budget is spent; its rate is scaled to the whole
stack, and its result is compared with the GPU's own input to the first
layer it did not reach (or the GPU's output, if it reached the end).

Prints one JSON line: tokens/s, the HBM roofline of the dominant kernel on
algorithmic (active) bytes, the active-byte rate of the whole step, and the
CPU oracle baseline.

Summary modes (no GPU): --summarize-trace turns a rocprofv3 kernel-trace CSV
into the per-kernel table kept under profiles/, and --summarize-traffic turns
a FETCH_SIZE and a WRITE_SIZE counter CSV into a per-launch traffic summary.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
MALL_BYTES = 256e6      # MI355X last-level (Infinity) cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=4, help="workload index (0..4)")
    ap.add_argument("--batch", type=int, default=1, help="sequences per decode step (1..32)")
    ap.add_argument("--layers", type=int, default=0, help="override the number of layers (0 = all)")
    ap.add_argument("--order", default="hot_first", choices=["hot_first", "identity"])
    ap.add_argument("--hot", default="0",
                    help="hot-dense prefix per layer: 0 (off), auto (the byte model's prefix, "
                         "workload.hot_count) or a slot count")
    ap.add_argument("--predictor-study", action="store_true",
                    help="CPU only: recall / precision of rank-r SVD predictors against the true "
                         "activations, for several singular spectra (activation_sparse_predict_amd.sizing)")
    ap.add_argument("--dense-sweep", action="store_true",
                    help="time the batched FFN (pi_sparse_ffn at --batch) over an explicit union of "
                         "growing size, gathered and dense, and print the table (one layer of --config)")
    ap.add_argument("--dense-frac", type=float, default=0.0,
                    help="batch > 1: union fraction from which the FFN runs over every neuron "
                         "(0 = the library's default, above 1 = never)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU oracle budget (the first layers of the first timed tokens); 0 = skip")
    ap.add_argument("--cpu-tokens", type=int, default=1, help="timed tokens the CPU oracle runs")
    ap.add_argument("--repeats", type=int, default=5, help="timed repeats; the median is reported")
    ap.add_argument("--eager", action="store_true",
                    help="launch the stack directly instead of replaying graphs (for counter runs)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run a plain elementwise copy of this many MiB (counter calibration)")
    ap.add_argument("--dump-counts", default="", help="write the per-token active counts here (JSON)")
    ap.add_argument("--summarize-trace", metavar="CSV", default="",
                    help="summarize a rocprofv3 kernel_trace.csv (no GPU); with --title, --command, --out")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COUNTS_JSON"),
                    help="summarize FETCH_SIZE / WRITE_SIZE counter CSVs of one kernel (no GPU); "
                         "with --kernel, --command, --out")
    ap.add_argument("--kernel", default="", help="kernel name for --summarize-traffic")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV", default=None,
                    help="per-launch means of rocprofv3 --pmc counter CSVs for --kernels")
    ap.add_argument("--kernels", default="", help="comma-separated kernel names for --summarize-counters")
    ap.add_argument("--trace", default="", help="kernel-trace CSV of the same program (--summarize-counters)")
    ap.add_argument("--source-rev", default="",
                    help="git revision whose HIP sources the counter run used (default: the working tree)")
    ap.add_argument("--title", default="", help="heading of a summary")
    ap.add_argument("--command", action="append", default=[], help="command line recorded in a summary")
    ap.add_argument("--out", default="", help="summary file to write (default: stdout)")
    return ap.parse_args()


def sizes(cfg):
    pb = {"f32": 4, "f16": 2}[cfg.p_dtype]
    wb = {"f32": 4.0, "f16": 2.0, "q4_0": 18.0 / 32.0}[cfg.w_dtype]
    n_mat = 3 if cfg.act == "reglu" else 2
    return pb, wb, n_mat


def kernel_bytes(cfg, batch, k, k_nz=None, hot=0):
    """Algorithmic HBM bytes of one launch of each kernel of a layer, k active (union) neurons.

    Dense predictor (A, B) and its bias, the active rows of gate/up with their
    bias, the rows of W_down^T that are read with their h values, and the x/y
    vectors of the glue.  At batch 1 the down projection reads only the k_nz
    active neurons whose h is nonzero; at batch > 1 every union row.  Rows of
    inactive neurons, scratch buffers and re-reads are not counted.  The
    per-kernel figures sum to the per-layer formula
    (r*d + f*r)*pb + 4f + k*((n_mat-1)*d*wb + 4) + k_nz*(d*wb + 4) + 8*d*B.
    With a hot-dense prefix of `hot` slots, only the tail's rows of B and
    predictor biases are read (f - hot rows at batch 1; at batch > 1 the
    score kernel's blocks of 32 * bscore_tiles(f) neurons not wholly inside the
    prefix), and k includes the prefix.
    """
    pb, wb, n_mat = sizes(cfg)
    d, f, r = cfg.d, cfg.ffn, cfg.rank
    n_up = n_mat - 1
    if k_nz is None:
        k_nz = k
    if batch == 1:
        fp = f - hot
        return {"k_predict_t": r * d * pb + 8 * d,
                "k_score": fp * r * pb + 4 * fp + k * (n_up * d * wb + 4),
                "k_down": k_nz * d * wb + 4 * k_nz}
    blk = 32 * bscore_tiles(f)                       # neurons per block of the batched score kernel
    fp = f - blk * (hot // blk)
    return {"k_bglue": 8 * d * batch, "k_bpred1": r * d * pb, "k_bsplit_t": 0,
            "k_bscore": fp * r * pb + 4 * fp, "k_compact": 0,
            "k_bup": k * (n_up * d * wb + 4), "k_bdown": k * d * wb + 4 * k}


def bscore_tiles(f):
    """32-neuron tiles per block of the batched score kernel: of 4, 3, 2, 1 the one
    with the fewest rounds of 256 blocks times tiles, the larger on a tie (the
    library's launch rule)."""
    best, nt = None, 4
    for t in (4, 3, 2, 1):
        cost = -(-(-(-f // (32 * t))) // 256) * t
        if best is None or cost < best:
            best, nt = cost, t
    return nt


def layer_bytes(cfg, k, batch=1, k_nz=None, hot=0):
    return float(sum(kernel_bytes(cfg, batch, k, k_nz, hot).values()))


def copy_bandwidth(torch, dev, stream, mib=1024, reps=5):
    """Device-copy bandwidth measured in this run: read + write bytes of a plain
    elementwise copy of `mib` MiB, per second (the median of `reps` copies)."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    times = []
    with torch.cuda.stream(stream):
        dst.copy_(src)
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
    del src, dst
    ms = sorted(times)[len(times) // 2]
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def source_digest(rev=None):
    """sha256 over the HIP sources (of the working tree, or of git revision `rev`);
    counter summaries taken on other sources do not apply."""
    import subprocess
    h = hashlib.sha256()
    csrc = "activation_sparse_predict_amd/csrc"
    if rev:
        names = subprocess.run(["git", "ls-tree", "--name-only", f"{rev}:{csrc}"], cwd=ROOT, check=True,
                               capture_output=True, text=True).stdout.split()
        for n in sorted(names):
            blob = subprocess.run(["git", "show", f"{rev}:{csrc}/{n}"], cwd=ROOT, check=True,
                                  capture_output=True).stdout
            h.update(n.encode() + b"\0" + blob)
        return h.hexdigest()
    for p in sorted(glob.glob(os.path.join(ROOT, csrc, "*"))):
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode() + b"\0" + fh.read())
    return h.hexdigest()


def counter_traffic(kernel, workload, batch):
    """HBM bytes per launch from a committed counter summary, or None.

    The summary under profiles/ carries machine-readable lines
    `kernel:`, `workload:`, `batch:`, `source_sha256:`,
    `traffic_bytes_per_launch:` and `alg_bytes_per_launch:`; it applies only
    while the HIP sources hash to the recorded digest.
    """
    digest = source_digest()
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))):
        kv = {}
        with open(p) as fh:
            for line in fh:
                m = re.match(r"^- ([a-z_0-9]+): `([^`]+)`$", line.strip())
                if m:
                    kv[m.group(1)] = m.group(2)
        if (kv.get("kernel") == kernel and kv.get("workload") == workload
                and kv.get("batch") == str(batch) and kv.get("source_sha256") == digest):
            return {"traffic": float(kv["traffic_bytes_per_launch"]),
                    "alg": float(kv["alg_bytes_per_launch"]), "file": os.path.relpath(p, ROOT)}
    return None


def _csv_rows(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _col(row, *names, default=None):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    return default


def _short(name):
    """Kernel name without its argument list."""
    return name.split("(")[0].strip()


def summarize_counters(paths, kernels, trace_csv, title, commands, out):
    """Per-launch means of every counter in rocprofv3 --pmc CSVs for each kernel whose
    name contains one of `kernels`; with a kernel-trace CSV of the same program, the
    MFMA rate SQ_INSTS_VALU_MFMA_MOPS_F16 * 512 flop per mean launch duration and its
    share of the dense fp16 peak (2.5 PFLOP/s)."""
    import statistics
    vals = {}
    for path in paths:
        for r in _csv_rows(path):
            kn = _short(_col(r, "Kernel_Name"))
            k = next((k for k in kernels if k in kn), None)
            if k is not None:
                vals.setdefault(k, {}).setdefault(_col(r, "Counter_Name"), []).append(float(_col(r, "Counter_Value")))
    dur = {}
    if trace_csv:
        for r in _csv_rows(trace_csv):
            kn = _short(_col(r, "Kernel_Name", "Name"))
            k = next((k for k in kernels if k in kn), None)
            if k is not None:
                dur.setdefault(k, []).append(float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp")))
    L = [f"# Counters: {title}", "", "Commands (from the repository root, on a machine with the GPU):", "", "```"]
    L += commands + ["```", "", "Summarized by `python bench.py --summarize-counters`: per-launch means.", ""]
    names = sorted({c for k in vals for c in vals[k]})
    L.append("| kernel | launches | " + " | ".join(names) + " | mean us | MFMA TFLOP/s (fp16) | of 2.5 PFLOP/s |")
    L.append("|---|---|" + "---|" * len(names) + "---|---|---|")
    for k in kernels:
        if k not in vals:
            continue
        v = vals[k]
        n = max(len(x) for x in v.values())
        row = [f"`{k}`", str(n)] + [f"{statistics.mean(v[c]):.4g}" if c in v else "" for c in names]
        us = statistics.mean(dur[k]) / 1e3 if dur.get(k) else None
        mops = statistics.mean(v["SQ_INSTS_VALU_MFMA_MOPS_F16"]) if "SQ_INSTS_VALU_MFMA_MOPS_F16" in v else None
        busy, gui = v.get("SQ_VALU_MFMA_BUSY_CYCLES"), v.get("GRBM_GUI_ACTIVE")
        row.append(f"{us:.2f}" if us else "")
        row.append(f"{mops * 512 / (us * 1e-6) / 1e12:.1f}" if (us and mops is not None) else "")
        row.append(f"{mops * 512 / (us * 1e-6) / 2.5e15:.3f}" if (us and mops is not None) else "")
        L.append("| " + " | ".join(row) + " |")
    text = "\n".join(L) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    else:
        print(text, end="")


def summarize_trace(path, title, commands, out):
    """Per-kernel table (calls, mean/median/min/max duration, share, launch shape,
    registers, LDS) from a rocprofv3 --kernel-trace CSV (one row per dispatch)."""
    import statistics
    rows = _csv_rows(path)
    agg, meta = {}, {}
    for r in rows:
        n = _short(_col(r, "Kernel_Name", "Name"))
        dur = float(_col(r, "End_Timestamp")) - float(_col(r, "Start_Timestamp"))
        agg.setdefault(n, []).append(dur)
        meta[n] = (_col(r, "Grid_Size_X", "Grid_Size", default="?"),
                   _col(r, "Workgroup_Size_X", "Workgroup_Size", default="?"),
                   _col(r, "Arch_VGPR_Count", "VGPR_Count", default="?"),
                   _col(r, "Accum_VGPR_Count", default="?"),
                   _col(r, "Group_Segment_Size", "LDS_Block_Size", default="?"),
                   _col(r, "Private_Segment_Size", "Scratch_Size", default="?"))
    total = sum(sum(v) for v in agg.values())
    L = [f"# Kernel trace: {title}", "", "Command (from the repository root, on a machine with the GPU):", "", "```"]
    L += commands + ["```", "",
                     f"Summarized by `python bench.py --summarize-trace` from the trace CSV of that run "
                     f"({len(rows)} dispatches).  Durations are end minus start timestamps of each dispatch.", "",
                     "| kernel | calls | avg us | median us | min us | max us | total ms | % | grid | wg | vgpr | agpr "
                     "| LDS_Block_Size | scratch B |",
                     "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for n, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        g, wg, vg, ag, lds, scr = meta[n]
        L.append(f"| `{n[:80]}` | {len(v)} | {statistics.mean(v) / 1e3:.2f} | {statistics.median(v) / 1e3:.2f} | "
                 f"{min(v) / 1e3:.2f} | {max(v) / 1e3:.2f} | {sum(v) / 1e6:.3f} | {100 * sum(v) / total:.1f} | "
                 f"{g} | {wg} | {vg} | {ag} | {lds} | {scr} |")
    stats = path.replace("kernel_trace.csv", "kernel_stats.csv")
    if stats != path and os.path.exists(stats):
        L += ["", f"rocprofv3's own `--stats` summary of the same run (`{os.path.basename(stats)}`, "
                  "durations in ns):", "", "```"]
        with open(stats) as fh:
            L += [line.rstrip("\n")[:400] for line in fh][:12]
        L.append("```")
    text = "\n".join(L) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    else:
        sys.stdout.write(text)


def summarize_traffic(fetch_csv, write_csv, counts_json, kernel, commands, out, source_rev=None):
    """HBM bytes per launch of one kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
    the calibration maps of known size (a plain elementwise map reading and writing
    calib_mb MiB), against the algorithmic bytes of the same launches."""
    import statistics

    import workload
    with open(counts_json) as fh:
        cj = json.load(fh)
    cfg = workload.CONFIGS[cj["config"]].with_(n_layers=cj["layers"])
    batch, calib_kib = cj["batch"], cj["calib_mb"] * 1024.0
    vals = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = {}
        for r in _csv_rows(path):
            kn = _col(r, "Kernel_Name")
            key = "calib" if "neg_kernel" in kn else (kernel if kernel in _short(kn) else None)
            if key is not None:
                per.setdefault(key, []).append(float(_col(r, "Counter_Value")))
        vals[name] = {k: (statistics.mean(v), len(v)) for k, v in per.items()}
    f_scale = calib_kib / vals["FETCH_SIZE"]["calib"][0]
    w_scale = calib_kib / vals["WRITE_SIZE"]["calib"][0]
    f_raw, n_launch = vals["FETCH_SIZE"][kernel]
    w_raw, _ = vals["WRITE_SIZE"][kernel]
    # every pass of the profiled program: the eager warm-up (token 0), then the tokens
    passes = [0] + list(range(len(cj["counts"])))
    hots = cj.get("hots", [0] * cj["layers"])
    alg = statistics.mean(kernel_bytes(cfg, batch, cj["counts"][t][l], cj["nz_counts"][t][l], hots[l])[kernel]
                          for t in passes for l in range(cj["layers"]))
    rd, wr = f_raw * f_scale * 1024, w_raw * w_scale * 1024
    tr = rd + wr
    L = [f"# HBM traffic of `{kernel}`, {cfg.name}, batch {batch}", "",
         "Two counter passes over the same program, from the repository root:", "", "```"]
    L += commands + ["```", "",
                     f"Summarized by `python bench.py --summarize-traffic`.  Calibration: the program first runs three "
                     f"plain elementwise maps that each read and write {cj['calib_mb']} MiB.  FETCH_SIZE read "
                     f"{vals['FETCH_SIZE']['calib'][0]:.0f} KiB and WRITE_SIZE {vals['WRITE_SIZE']['calib'][0]:.0f} KiB "
                     f"per map (expected {calib_kib:.0f} KiB each), so the kernel's counters are scaled by "
                     f"{f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
                     "Algorithmic bytes: the per-launch byte model of the benchmark (`kernel_bytes`), with the active "
                     "counts of every (pass, layer) of the same run.", "",
                     "| | per launch |", "|---|---|",
                     f"| launches profiled | {n_launch} |",
                     f"| FETCH_SIZE raw | {f_raw:.1f} KiB |",
                     f"| WRITE_SIZE raw | {w_raw:.1f} KiB |",
                     f"| HBM read (scaled) | {rd / 1e6:.3f} MB |",
                     f"| HBM write (scaled) | {wr / 1e6:.3f} MB |",
                     f"| traffic | {tr / 1e6:.3f} MB |",
                     f"| algorithmic bytes (same launches) | {alg / 1e6:.3f} MB |",
                     f"| traffic / algorithmic | {tr / alg:.4f} |", "",
                     "Machine-readable (read by the benchmark, which reports the traffic only while the HIP",
                     "sources hash to the digest below):", "",
                     f"- kernel: `{kernel}`",
                     f"- workload: `{workload.CONFIGS[cj['config']].name}`",
                     f"- batch: `{batch}`",
                     f"- source_sha256: `{source_digest(source_rev)}`",
                     f"- traffic_bytes_per_launch: `{tr:.1f}`",
                     f"- alg_bytes_per_launch: `{alg:.1f}`"]
    text = "\n".join(L) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    else:
        sys.stdout.write(text)


def dense_sweep(args):
    """Gathered against dense batched FFN on one layer: for union fractions u, an
    explicit ascending union of round(u f) random neurons, each sequence's mask a
    random half of it; pi_sparse_ffn with dense_frac above 1 (gathered rows) and
    tiny (every neuron), the median of `reps` timed calls each."""
    import numpy as np
    import torch
    import activation_sparse_predict_amd as pi
    import workload
    cfg = workload.CONFIGS[args.config]
    B = max(2, args.batch)
    dev = torch.device("cuda:0")
    lw = workload.make_layer(cfg, 0, nthreads=16)
    L = pi.DeviceLayer.upload(lw, dev)
    del lw
    f, d = cfg.ffn, cfg.d
    rng = np.random.default_rng(7)
    x = torch.from_numpy(workload.make_x(cfg, 0, seqs=B)).to(dev)
    y = torch.empty(B, d, device=dev)
    ws = pi.alloc_workspace(L, B)
    stream = torch.cuda.current_stream()
    _, wb, n_mat = sizes(cfg)
    rows = []
    for u in (0.3, 0.5, 0.7, 0.8, 0.9, 0.95, 1.0):
        k = max(1, int(round(u * f)))
        idx = np.sort(rng.choice(f, size=k, replace=False)).astype(np.int32)
        mask = np.zeros((B, f), np.uint8)
        mask[:, idx] = rng.random((B, k)) < 0.5
        idx_t = torch.from_numpy(idx).to(dev)
        cnt_t = torch.tensor([k], dtype=torch.int32, device=dev)
        mask_t = torch.from_numpy(mask).to(dev)
        res = {}
        for tag, frac in (("gathered", 2.0), ("dense", 1e-6)):
            L.struct.dense_frac = frac
            for _ in range(3):
                pi.sparse_ffn(L, x, idx_t, cnt_t, y, mask=mask_t, ws=ws, batch=B)
            times = []
            for _ in range(args.repeats * 4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                pi.sparse_ffn(L, x, idx_t, cnt_t, y, mask=mask_t, ws=ws, batch=B)
                e1.record(stream)
                e1.synchronize()
                times.append(e0.elapsed_time(e1) * 1e3)
            res[tag] = sorted(times)[len(times) // 2]
        ub = k * (n_mat * d * wb + 8)
        rows.append((u, k, res["gathered"], res["dense"], ub / res["gathered"] / 1e3, ub / res["dense"] / 1e3))
        log(f"[sweep] union {u:.2f} ({k} of {f}): gathered {res['gathered']:.1f} us, dense {res['dense']:.1f} us")
    print(f"# batched FFN, {cfg.name}, batch {B}: pi_sparse_ffn over an explicit union, median us")
    print("| union | rows | gathered us | dense us | gathered GB/s (union bytes) | dense GB/s (union bytes) |")
    print("|---|---|---|---|---|---|")
    for u, k, g, dn, gg, dg in rows:
        print(f"| {u:.2f} | {k} | {g:.1f} | {dn:.1f} | {gg:.0f} | {dg:.0f} |")


def main():
    args = parse()
    if args.predictor_study:
        from activation_sparse_predict_amd import sizing
        t0 = time.time()
        for d, f in ((1024, 4096), (4096, 11008)):
            rows = sizing.study(d=d, f=f, ranks=(16, 64, 256, 1024), alphas=(0.0, 0.5, 1.0))
            print(f"# predictor sizing, d={d}, f={f}, mean firing rate 0.1, 256 tokens (fp16 predictor and up)")
            print(sizing.table(rows))
            print()
        log(f"[study] {time.time() - t0:.1f} s")
        return
    if args.dense_sweep:
        dense_sweep(args)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.title or args.summarize_trace, args.command, args.out)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, [k for k in args.kernels.split(",") if k], args.trace,
                           args.title, args.command, args.out)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.kernel, args.command, args.out, args.source_rev)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on exactly one GPU (asked for {args.gpus}); "
              "the sparse FFN is not sharded across GPUs here.", file=sys.stderr)
        sys.exit(2)
    B = args.batch
    if not 1 <= B <= 32:
        print("bench.py: --batch must be in 1..32", file=sys.stderr)
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
    W, K, L = args.warmup, args.steps, cfg.n_layers
    kernels = pi.LAYER_KERNELS[1 if B == 1 else 2]
    log(f"[bench] {cfg.name}: L={L} d={cfg.d} f={cfg.ffn} r={cfg.rank} "
        f"{cfg.w_dtype}/{cfg.p_dtype} {cfg.act}; batch {B}; warmup {W}, steps {K}")

    stream = torch.cuda.Stream()
    if args.calib_copy_mb:
        # a plain elementwise map (read n bytes, write n bytes) for counter calibration
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(stream):
            for _ in range(3):
                torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: 3 x {args.calib_copy_mb} MiB read + write")
        del src, dst

    xs_host = workload.make_tokens(cfg, W + K, seqs=B)              # [W+K][B][d] float32

    # ---- weights: generated on the host one layer at a time and uploaded; the
    # CPU oracle runs layer-major on the same host layer before it is dropped,
    # on the first timed token(s), until its budget is spent (only the oracle's
    # own work is timed, not the generation)
    import oracle
    t0 = time.time()
    layers = []
    cpu_seqs = [(W + t, b) for t in range(K) for b in range(B)][:max(1, args.cpu_tokens)]
    x_cpu = np.stack([xs_host[t][b] for t, b in cpu_seqs]).astype(np.float64) if args.cpu_seconds > 0 else None
    cpu_time, cpu_layers = 0.0, 0
    hots = []
    for l in range(L):
        lw = workload.make_layer(cfg, l, order=args.order, nthreads=nthr)
        lw.hot = workload.hot_count(cfg, lw.p_storage) if args.hot == "auto" else int(args.hot)
        lw.dense_frac = args.dense_frac
        hots.append(lw.hot)
        layers.append(pi.DeviceLayer.upload(lw, dev))
        if x_cpu is not None and cpu_layers == l and cpu_time < args.cpu_seconds:
            tc0 = time.perf_counter()
            r = oracle.layer_forward(lw, x_cpu)
            x_cpu = oracle.rms_glue(x_cpu, r["y"])
            cpu_time += time.perf_counter() - tc0
            cpu_layers += 1
        del lw
        if (l + 1) % 8 == 0 and l + 1 < L:
            log(f"[bench]   layer {l + 1}/{L} generated ({time.time() - t0:.0f} s; oracle through "
                f"{cpu_layers} layers, {cpu_time:.1f} s)")
    torch.cuda.synchronize()
    wbytes = sum(Ld.nbytes() for Ld in layers)
    log(f"[bench] generated + uploaded {wbytes / 1e9:.2f} GB in {time.time() - t0:.1f} s")

    xs = torch.from_numpy(np.ascontiguousarray(xs_host)).to(dev)
    outs = torch.empty_like(xs)
    counts = torch.zeros((W + K, L), dtype=torch.int32, device=dev)
    nz_counts = torch.zeros((W + K, L), dtype=torch.int32, device=dev)   # rows of W_down^T read
    stack = pi.Stack(layers, batch=B)

    # ---- every EVERY-th token slot carries events on one layer, in pairs of
    # slots on the same layer: a "full" slot brackets each kernel of the layer,
    # the next an "ends" slot brackets only the whole layer.  An event node adds
    # a cost c to each interval, so (sum of full intervals - ends interval) =
    # (kernels - 1) c.
    n_ev = len(kernels) + 1
    EVERY = 4
    events, traces, ev_layer, ev_full = {}, {}, {}, {}
    for t in range(W + K):
        if t % EVERY:
            traces[t] = None
            continue
        pidx = t // EVERY
        l = (7 * (pidx // 2)) % L
        full = pidx % 2 == 0
        evs = [pi.HipEvent() if (full or i in (0, n_ev - 1)) else None for i in range(n_ev)]
        recs = [dict() for _ in range(L)]
        recs[l] = {"events": [int(e) if e is not None else 0 for e in evs]}
        events[t], ev_layer[t], ev_full[t] = evs, l, full
        traces[t] = pi.make_trace(L, recs)

    def run_token(t, s):
        stack(xs[t], outs[t], counts[t], traces[t], stream=s, nz_counts=nz_counts[t])

    run_token(0, stream)                                           # eager warm-up of the path
    stream.synchronize()
    graphs = []
    if not args.eager:
        for t in range(W + K):
            graphs.append(pi.HipGraph(stream, lambda s, t=t: run_token(t, s)))
        torch.cuda.synchronize()
        log(f"[bench] captured {len(graphs)} token graphs")

    def replay(t):
        if args.eager:
            run_token(t, stream)
        else:
            graphs[t].replay()

    times = []
    kdur = {k: [] for k in kernels}      # ms per launch
    kbytes = {k: [] for k in kernels}    # algorithmic bytes of the same launches
    pair_full, pair_ends = {}, {}        # per (repeat, pair): sum of kernel intervals / whole layer
    ev0, ev1 = pi.HipEvent(), pi.HipEvent()
    for rep in range(args.repeats):
        for t in range(W):
            replay(t)
        torch.cuda.synchronize()
        ev0.record(stream)
        for t in range(W, W + K):
            replay(t)
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_ms(ev1)
        times.append(ms)
        cnt_rep = counts.cpu().numpy()
        nz_rep = nz_counts.cpu().numpy()
        for t in range(W, W + K):
            if t not in events:
                continue
            evs, key = events[t], (rep, t // (2 * EVERY))
            if not ev_full[t]:
                pair_ends[key] = evs[0].elapsed_ms(evs[n_ev - 1])
                continue
            kb = kernel_bytes(cfg, B, int(cnt_rep[t, ev_layer[t]]), int(nz_rep[t, ev_layer[t]]), hots[ev_layer[t]])
            iv = [evs[i].elapsed_ms(evs[i + 1]) for i in range(len(kernels))]
            pair_full[key] = sum(iv)
            for i, k in enumerate(kernels):
                kdur[k].append(iv[i])
                kbytes[k].append(kb[k])
        log(f"[bench] repeat {rep}: {K} steps in {ms:.3f} ms ({B * K / ms * 1e3:.1f} tok/s)")
    ms = float(np.median(times))
    ms_per_step = ms / K

    cnt = counts[W:].cpu().numpy().astype(np.int64)                # [K][L]
    cnt_nz = nz_counts[W:].cpu().numpy().astype(np.int64)
    if args.dump_counts:
        with open(args.dump_counts, "w") as fh:
            json.dump({"workload": cfg.name, "config": args.config, "layers": L, "batch": B,
                       "warmup": W, "steps": K, "repeats": args.repeats, "calib_mb": args.calib_copy_mb,
                       "counts": counts.cpu().numpy().tolist(),
                       "nz_counts": nz_counts.cpu().numpy().tolist(), "hots": hots}, fh)
    step_bytes = float(sum(layer_bytes(cfg, int(cnt[t, l]), B, int(cnt_nz[t, l]), hots[l])
                           for t in range(K) for l in range(L))) / K
    stack_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    copy_gbs = copy_bandwidth(torch, dev, stream)
    log(f"[bench] device copy in this run: {copy_gbs:.1f} GB/s (read + write); the step reaches "
        f"{stack_gbs / copy_gbs:.3f} of it")
    mean_active = float(cnt.mean() / cfg.ffn)
    nz_share = float(cnt_nz.sum() / max(cnt.sum(), 1))
    log(f"[bench] mean active {mean_active:.4f} (h != 0: {nz_share:.3f} of them), {step_bytes / 1e6:.2f} MB/step, "
        f"{stack_gbs:.1f} GB/s over the whole step ({stack_gbs / HBM_PEAK_GBS:.3f} of peak)")

    # ---- per-kernel durations sampled over the timed region, less the event-node cost
    per_kernel = {}
    pairs = sorted(set(pair_full) & set(pair_ends))
    raw_layer_us = float(np.mean([pair_full[p] for p in pairs])) * 1e3 if pairs else 0.0
    ends_layer_us = float(np.mean([pair_ends[p] for p in pairs])) * 1e3 if pairs else 0.0
    node_us = max(0.0, (raw_layer_us - ends_layer_us) / (len(kernels) - 1)) if pairs else 0.0
    for k in kernels:
        raw = np.asarray(kdur[k]) * 1e3
        d_us = np.maximum(raw - node_us, 1e-3)
        b = np.asarray(kbytes[k], dtype=np.float64)
        per_kernel[k] = {"avg_us": float(d_us.mean()), "raw_interval_us": float(raw.mean()),
                         "launches": int(d_us.size), "alg_bytes_per_launch": float(b.mean()),
                         "gbs": float(b.sum() / (d_us.sum() * 1e-6) / 1e9) if b.sum() else 0.0}
        log(f"[bench]   {k:12s} {per_kernel[k]['avg_us']:8.2f} us (interval {raw.mean():6.2f})  "
            f"{per_kernel[k]['alg_bytes_per_launch'] / 1e6:8.3f} MB  {per_kernel[k]['gbs']:8.1f} GB/s")
    layer_us = sum(v["avg_us"] for v in per_kernel.values())
    log(f"[bench]   event node cost {node_us:.2f} us per interval ({len(pairs)} layer pairs: kernel intervals "
        f"{raw_layer_us:.2f} us, whole layer {ends_layer_us:.2f} us; step/L {ms_per_step * 1e3 / L:.2f} us)")
    dom = max(kernels, key=lambda k: per_kernel[k]["avg_us"])
    dk = per_kernel[dom]
    tr = counter_traffic(dom, cfg.name, B)
    traffic = None
    if tr is not None:
        # counters are per launch of the profiled run; scale to this run's launches
        traffic = tr["traffic"] / tr["alg"] * dk["alg_bytes_per_launch"]

    # ---- CPU oracle: the layers it ran, scaled to the whole stack, and its
    # result against the GPU's own input to the next layer (or the GPU output)
    cpu = None
    if x_cpu is not None and cpu_layers > 0:
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = 1
        if cpu_layers == L:
            gpu_x = np.stack([outs[t][b].cpu().numpy() for t, b in cpu_seqs])
            where = "the GPU stack output"
        else:
            # the GPU's input to layer cpu_layers for the same token(s): one traced pass
            xin = torch.empty((B, cfg.d), dtype=torch.float32, device=dev)
            recs = [dict() for _ in range(L)]
            recs[cpu_layers] = {"x_in": xin}
            gpu_x = []
            for t in sorted({t for t, _ in cpu_seqs}):
                stack(xs[t], torch.empty_like(outs[t]), None, pi.make_trace(L, recs), stream=stream)
                stream.synchronize()
                gpu_x += [xin[b].cpu().numpy() for tt, b in cpu_seqs if tt == t]
            gpu_x = np.stack(gpu_x)
            where = f"the GPU's input to layer {cpu_layers}"
        err = max(float(np.abs(gpu_x[i] - x_cpu[i]).max() / max(np.abs(x_cpu[i]).max(), 1e-30))
                  for i in range(len(cpu_seqs)))
        n_tok = len(cpu_seqs)
        scaled_s = cpu_time * L / cpu_layers
        cpu = {"value": n_tok / scaled_s, "unit": "tokens/s", "cores": int(blas_threads),
               "kind": "oracle",
               "sample": f"{n_tok} sequence-token(s) of the first timed step through the first {cpu_layers} of "
                         f"{L} layers, layer-major, float64 NumPy oracle, {cpu_time:.1f} s of oracle work "
                         f"(generation not timed), scaled to all {L} layers",
               "host_cores_visible": os.cpu_count(),
               "host_cores_affinity": len(os.sched_getaffinity(0)),
               "threads_note": "cores = threads of the BLAS pool the oracle's products ran on",
               "max_rel_err_vs_gpu": err, "compared_with": where}
        log(f"[bench] oracle: {n_tok} token(s) through {cpu_layers}/{L} layers in {cpu_time:.1f} s "
            f"({cpu['value']:.4f} tokens/s scaled to the stack); max rel err against {where} {err:.2e}")

    metric = ("sparse-FFN tokens/s at batch 1 (1 GPU); active-byte HBM GB/s vs peak" if B == 1
              else f"sparse-FFN tokens/s at batch {B} (1 GPU); active-byte HBM GB/s vs peak")
    res = {
        "metric": metric,
        "value": B * K / (ms * 1e-3),
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
        "config": {"workload": cfg.name, "layers": L, "d": cfg.d, "ffn": cfg.ffn,
                   "rank": cfg.rank, "batch": B, "act": cfg.act, "w_dtype": cfg.w_dtype,
                   "p_dtype": cfg.p_dtype, "order": args.order, "hot_prefix": args.hot,
                   "dense_frac": args.dense_frac,
                   "hot_mean": float(np.mean(hots)), "mean_active": mean_active,
                   "down_rows_read_share": nz_share,
                   "graphs": not args.eager, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": dk["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dk["gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "frac_of_measured_copy": dk["gbs"] / copy_gbs,
                     "kernel": dom, "avg_launch_us": dk["avg_us"],
                     "alg_bytes_per_launch": dk["alg_bytes_per_launch"],
                     "launches_timed": dk["launches"], "event_node_us_subtracted": node_us,
                     "traffic_unit": "HBM bytes per launch (counter summary "
                                     + (tr["file"] if tr else "absent or stale") + ")"},
        "stack_hbm": {"achieved": stack_gbs, "frac": stack_gbs / HBM_PEAK_GBS, "unit": "GB/s",
                      "copy_gbs_measured": copy_gbs, "frac_of_copy": stack_gbs / copy_gbs,
                      # a step that moves less than the 256 MB last-level cache (MALL) is served
                      # from cache, not HBM: its fraction of the HBM peak means nothing
                      "cache_resident": step_bytes < MALL_BYTES,
                      "alg_bytes_per_step": step_bytes},
        "kernels": per_kernel,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
