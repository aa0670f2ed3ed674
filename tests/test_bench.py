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
