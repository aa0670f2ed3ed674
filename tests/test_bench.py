"""Host-side checks of the benchmark's byte accounting and argument contract (no GPU)."""
import os
import subprocess
import sys

import pytest

import bench
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def layer_formula(cfg, k, k_nz, batch=1):
    """(r*d + f*r)*pb + 4f + k*((n_mat-1)*d*wb + 4) + k_nz*(d*wb + 4) + 8*d*batch."""
    pb, wb, n_mat = bench.sizes(cfg)
    d, f, r = cfg.d, cfg.ffn, cfg.rank
    return (r * d + f * r) * pb + 4 * f + k * ((n_mat - 1) * d * wb + 4) + k_nz * (d * wb + 4) + 8 * d * batch


@pytest.mark.parametrize("ci", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("batch", [1, 8, 32])
def test_kernel_bytes_add_up_to_the_layer_formula(ci, batch):
    cfg = workload.CONFIGS[ci]
    k = int(cfg.mean_active * cfg.ffn)
    k_nz = k // 3 if batch == 1 else k          # batched: every union row is read
    parts = bench.kernel_bytes(cfg, batch, k, k_nz)
    assert sum(parts.values()) == pytest.approx(layer_formula(cfg, k, k_nz, batch), rel=1e-12)
    assert bench.layer_bytes(cfg, k, batch, k_nz) == pytest.approx(sum(parts.values()), rel=1e-12)


def test_rows_read_default_to_the_active_count():
    cfg = workload.CONFIGS[1]
    assert bench.kernel_bytes(cfg, 1, 1000) == bench.kernel_bytes(cfg, 1, 1000, 1000)
    # fewer down rows read, fewer bytes, and only in the down projection
    a, b = bench.kernel_bytes(cfg, 1, 1000), bench.kernel_bytes(cfg, 1, 1000, 400)
    assert a["k_predict_t"] == b["k_predict_t"] and a["k_score"] == b["k_score"]
    assert a["k_down"] - b["k_down"] == 600 * (cfg.d * 2 + 4)


def test_llama7b_bytes_per_token_at_the_target_activity():
    # 32 layers at the 12% target mean with every active row read: 2.031 GB per token
    cfg = workload.CONFIGS[1]
    k = round(0.12 * cfg.ffn)
    assert 32 * bench.layer_bytes(cfg, k) / 1e9 == pytest.approx(2.031, abs=1e-3)


def test_q4_bytes_per_weight():
    pb, wb, n_mat = bench.sizes(workload.CONFIGS[4])
    assert (pb, wb, n_mat) == (2, 18 / 32, 2)      # fp16 predictor; 16 B of nibbles + 2 B scale per 32 weights


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_trace(tmp_path):
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X",
           "Arch_VGPR_Count", "Accum_VGPR_Count", "Group_Segment_Size", "Private_Segment_Size"]
    rows = [["void pik::k_score<1, 2>(int)", 1000, 3000, 131072, 256, 124, 0, 33072, 0],
            ["void pik::k_score<1, 2>(int)", 5000, 9000, 131072, 256, 124, 0, 33072, 0],
            ["pik::k_down(int)", 9000, 10000, 65536, 512, 72, 0, 66624, 0]]
    p = tmp_path / "kt.csv"
    _write_csv(p, hdr, rows)
    out = tmp_path / "s.md"
    bench.summarize_trace(str(p), "test", ["cmd"], str(out))
    text = out.read_text()
    line = [l for l in text.splitlines() if "k_score" in l][0].split("|")
    assert line[2].strip() == "2" and line[3].strip() == "3.00"            # calls, mean of 2 and 4 us
    assert line[5].strip() == "2.00" and line[6].strip() == "4.00"        # min, max
    assert "k_down" in text and "| 1 | 1.00 |" in text


def test_summarize_traffic(tmp_path):
    import json
    cfg = workload.CONFIGS[1].with_(n_layers=2)
    counts = [[100, 200], [300, 400]]
    nz = [[50, 60], [70, 80]]
    cj = tmp_path / "c.json"
    cj.write_text(json.dumps({"config": 1, "layers": 2, "batch": 1, "calib_mb": 1024, "counts": counts,
                              "nz_counts": nz}))
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the fetch counter reads half of the calibration map's bytes: scale 2; other
    # elementwise kernels of the program (fills) are not the calibration map
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"
    fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
    _write_csv(tmp_path / "f.csv", hdr, [[neg, "FETCH_SIZE", 524288]] * 3 + [[fill, "FETCH_SIZE", 7.0]] +
               [["void pik::k_down<1, 4, false>(int)", "FETCH_SIZE", 1000.0]] * 6)
    _write_csv(tmp_path / "w.csv", hdr, [[neg, "WRITE_SIZE", 1048576]] * 3 + [[fill, "WRITE_SIZE", 9.0]] +
               [["void pik::k_down<1, 4, false>(int)", "WRITE_SIZE", 10.0]] * 6)
    out = tmp_path / "t.md"
    bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(cj), "k_down", ["c"], str(out))
    kv = dict(l[2:].split(": ", 1) for l in out.read_text().splitlines() if l.startswith("- "))
    assert float(kv["traffic_bytes_per_launch"].strip("`")) == pytest.approx((2000 + 10) * 1024)
    # passes: token 0 (warm-up), then tokens 0 and 1; layers 0 and 1
    alg = [bench.kernel_bytes(cfg, 1, counts[t][l], nz[t][l])["k_down"] for t in (0, 0, 1) for l in (0, 1)]
    assert float(kv["alg_bytes_per_launch"].strip("`")) == pytest.approx(sum(alg) / len(alg))


def test_hot_prefix_bytes():
    """A hot-dense prefix drops its rows of B and predictor biases from the score
    kernel's bytes (batch 1: every prefix slot; batch > 1: whole blocks of 128 or 32 neurons)."""
    cfg = workload.CONFIGS[4]
    pb = 2
    a, b = bench.kernel_bytes(cfg, 1, 4000, 3900), bench.kernel_bytes(cfg, 1, 4000, 3900, hot=1109)
    assert a["k_score"] - b["k_score"] == 1109 * (cfg.rank * pb + 4)
    assert a["k_down"] == b["k_down"] and a["k_predict_t"] == b["k_predict_t"]
    a, b = bench.kernel_bytes(cfg, 32, 5000), bench.kernel_bytes(cfg, 32, 5000, hot=77)
    assert a["k_bscore"] == b["k_bscore"]
    a, b = bench.kernel_bytes(cfg, 32, 5000), bench.kernel_bytes(cfg, 32, 5000, hot=300)
    assert bench.bscore_tiles(cfg.ffn) == 3                  # 512 blocks of 96 neurons
    assert a["k_bscore"] - b["k_bscore"] == 288 * (cfg.rank * pb + 4)
    # narrower ffns: blocks of 64 neurons (172 blocks) and of 128 (256 blocks)
    c1 = workload.CONFIGS[1]
    assert bench.bscore_tiles(c1.ffn) == 2 and bench.bscore_tiles(workload.CONFIGS[3].ffn) == 4
    a, b = bench.kernel_bytes(c1, 32, 5000), bench.kernel_bytes(c1, 32, 5000, hot=77)
    assert a["k_bscore"] - b["k_bscore"] == 64 * (c1.rank * bench.sizes(c1)[0] + 4)

