"""Host checks of bench.py's bookkeeping (no GPU): the algorithmic bytes and flops behind `value`
and `roofline`, the roofline floor, the counter-traffic lookup and the one-GPU guard.

The expected figures are the per-configuration table of the verify-attention workload statement
(KV bytes, algorithmic bytes = KV + indices + mask + Q + out + lse, flops = q_len * H * L * 2176,
T* = max(bytes / 8 TB/s, flops / 2.5 PFLOP/s)), printed there to three significant digits.
"""
import hashlib
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402

# config: (KV MB, algorithmic MB, GFLOP, T* us)
TABLE = {
    "tiny_256_h8": (0.305, 0.466, 0.042, 0.06),
    "4k_h64": (4.73, 6.04, 5.15, 2.06),
    "16k_h64": (18.9, 20.4, 20.6, 8.22),
    "65k_h8": (75.5, 76.5, 10.3, 9.56),
    "ragged4_185k_h64": (394.0, 410.0, 762.0, 305.0),
}


def _shape(name):
    w = W.CONFIGS[name]
    return types.SimpleNamespace(prefixes=w.prefixes, q_len=w.q_len, B=w.B, H=w.H)


def _close(got, want):
    # the table rounds to three significant digits (0.06 us to one); allow one unit of its last digit
    digits = 1 if want < 0.1 else 3
    scale = 10 ** (digits - 1 - int(f"{want:e}".split("e")[1]))
    return abs(round(got * scale) / scale - want) <= 1.0 / scale + 1e-9


@pytest.mark.parametrize("name", sorted(TABLE))
def test_algorithmic_figures_match_the_workload_table(name):
    kv_mb, alg_mb, gflop, t_us = TABLE[name]
    a = bench.algorithmic(_shape(name))
    assert _close(a["kv_bytes"] / 1e6, kv_mb), (a["kv_bytes"], kv_mb)
    assert _close(a["step_bytes"] / 1e6, alg_mb), (a["step_bytes"], alg_mb)
    assert _close(a["flops"] / 1e9, gflop), (a["flops"], gflop)
    assert _close(bench.step_floor_us(a), t_us), (bench.step_floor_us(a), t_us)


def test_bound_follows_the_ridge():
    # 65k/H=8 sits below the 312 flop/B ridge (HBM-bound), the ragged batch far above it (MFMA-bound)
    for name, hbm_bound in (("65k_h8", True), ("ragged4_185k_h64", False)):
        a = bench.algorithmic(_shape(name))
        t_hbm = a["step_bytes"] / (bench.HBM_PEAK_GBS * 1e9) * 1e6
        t_mfma = a["flops"] / (bench.MFMA_BF16_PEAK_TFS * 1e12) * 1e6
        assert (t_hbm > t_mfma) == hbm_bound
        assert bench.step_floor_us(a) == max(t_hbm, t_mfma)


def _write_summary(root, sha):
    os.makedirs(os.path.join(root, "profiles"))
    t = {"source_sha256": sha, "fetch_kib_per_dispatch": 1000.0, "write_kib_per_dispatch": 200.0,
         "copy_fetch_factor": 0.5, "copy_write_factor": 1.0}
    with open(os.path.join(root, "profiles", "traffic_verify_partial_cfg_u7.json"), "w") as f:
        json.dump(t, f)


def test_measured_traffic_is_copy_scaled_and_tied_to_the_kernel_source(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel source v1\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    root = str(tmp_path / "repo")
    _write_summary(root, sha)
    monkeypatch.setattr(bench, "ROOT", root)
    traffic, where = bench.measured_traffic("cfg", "u7")
    # FETCH reads 0.5x and WRITE 1.0x of the bytes a plain copy moves
    assert traffic == 1000.0 * 1024 / 0.5 + 200.0 * 1024 / 1.0
    assert where.endswith("traffic_verify_partial_cfg_u7.json")
    # a changed kernel source voids the figure
    src.write_text("kernel source v2\n")
    assert bench.measured_traffic("cfg", "u7") == (None, "kernel changed since the counters were taken")
    assert bench.measured_traffic("other", "u7") == (None, "no counter summary")


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                          "--warmup", "0"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
