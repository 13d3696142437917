"""Host-side checks of bench.py: the one-GPU contract, the algorithmic byte
models the roofline divides by (against counts written out by hand), and the
rule that counter traffic is only reported for the source it was taken on."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_gdn_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_verify_bytes_chain8_by_hand():
    d = W.WORKLOADS["chain8-b1-h8-d256"](0)
    state = 8 * 256 * 256 * 4                 # FP32 state of 8 heads
    qkv = 8 * 8 * (256 + 256 + 256) * 2       # bf16 q, k, v of 8 nodes x 8 heads
    bg = 8 * 8 * 2 * 4                        # beta, g
    out = 8 * 8 * 256 * 4                     # FP32 outputs
    rec = 8 * 8 * (256 * 4 + 4 + 256 * 2) + 8 * (4 + 8)  # u', G, k copy; parents, masks
    assert bench.bytes_verify(d, tree=False) == state + qkv + bg + out + rec == 2360160
    assert bench.bytes_verify(d, tree=True) == 2360160 + 8 * 4  # plus the parent array


def test_commit_and_delayed_bytes_by_hand():
    d = W.WORKLOADS["tree32-b1-h8-d256"](0)
    H, dk, dv, N = 8, 256, 256, 32
    for n in (0, 1, 3):
        path = H * n * (dv * 4 + dk * 2 + 4)  # u', k (bf16), G of the path nodes
        commit = (2 * H * dv * dk * 4 + path + N * 8) if n else 0
        assert bench.bytes_commit(d, np.array([n])) == commit + 4
        delayed = bench.bytes_verify(d, True) + N * 8 + 4 + ((H * dv * dk * 4 + path) if n else 0)
        assert bench.bytes_delayed(d, np.array([n]), True) == delayed


def test_counter_traffic_needs_the_current_source(tmp_path, monkeypatch):
    kern, wl = "gdn_tree_verify", "tree32-b1-h8-d256"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = prof / f"traffic_{kern}_{wl}.txt"
    assert bench.measured_traffic(kern, wl) is None  # no summary
    f.write_text("# header\nhbm_bytes_per_launch: 12345\nsource_digest: 000000000000\n")
    assert bench.measured_traffic(kern, wl) is None  # taken on other code
    f.write_text(f"hbm_bytes_per_launch: 12345\nsource_digest: {bench.source_digest(kern)}\n")
    assert bench.measured_traffic(kern, wl) == 12345.0


def test_mfma_counters_need_the_current_source(tmp_path, monkeypatch):
    kern, wl = "gdn_tree_verify", "tree64-b8-h8-d256"
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = prof / f"mfma_{kern}_{wl}.txt"
    assert bench.measured_mfma(kern, wl, 10.0) is None  # no summary
    body = "bf16_mfma_flop_per_launch: 1000000000\nmfma_busy_cycles_per_simd: 1200\n"
    f.write_text(body + "source_digest: 000000000000\n")
    assert bench.measured_mfma(kern, wl, 10.0) is None  # taken on other code
    f.write_text(body + f"source_digest: {bench.source_digest(kern)}\n")
    m = bench.measured_mfma(kern, wl, 10.0)
    # 1 GFLOP in 10 us = 100 TFLOP/s = 4% of 2.5 PFLOP/s; 1200 of the
    # 24000 cycles of 10 us at 2.4 GHz = 5% busy
    assert m["issued_tflops"] == 100.0 and m["issued_frac"] == 0.04
    assert m["busy_cycles_per_simd"] == 1200.0 and m["busy_frac_at_2p4ghz"] == 0.05
