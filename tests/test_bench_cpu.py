"""CPU checks of bench.py's host side: the entry point exists, refuses more than one GPU with a
message, counts FLOPs by the metric's rule, and turns counter CSVs into the traffic record."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from context_blockwise_causal_amd import api  # noqa: E402


def test_entry_point_and_single_gpu_refusal():
    assert callable(bench.main)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counted_flops_rule():
    # contiguous cp=4: rank 2 sees 2 full chunks and its diagonal; 4 d L^2 per full, 2 d L^2 per diag
    prob = api.Problem(2, 4096, 12, 12, 64, 4, "contiguous", "bf16")
    L, d = 1024, 64
    f = bench.counted_flops(api, prob, 2)
    assert sum(f) == (2 * 4 * d * L * L + 2 * d * L * L) * 2 * 12
    # zigzag cp=8 rank 0: 15 full half-chunk pairs and 2 diagonal ones per the step rule
    prob = api.Problem(1, 32768, 32, 8, 128, 8, "zigzag", "bf16")
    L, d = 2048, 128
    assert sum(bench.counted_flops(api, prob, 0)) == (15 * 4 * d * L * L + 2 * 2 * d * L * L) * 32


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    def write(dirname, counter, rows):
        d = tmp_path / dirname
        d.mkdir()
        with open(d / "p_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for i, (k, v) in enumerate(rows):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})
        return str(d)
    calib = 1 << 20
    stage = 1 << 16
    # an earlier layout dispatch gathers a tensor of another size; the calibration is the last one
    fdir = write("f", "FETCH_SIZE", [("ra::layout_kernel(...)", calib / 1024 / 8),
                                     ("ra::layout_kernel(...)", calib / 1024 / 2),
                                     ("void ra::chunk_bwd_kv_pp_kernel<128, true>(ra::KParams)", 100.0),
                                     ("void ra::chunk_bwd_kv_pp_kernel<128, true>(ra::KParams)", 300.0),
                                     ("ra::copy2d_kernel(...)", stage / 1024 / 3)])
    wdir = write("w", "WRITE_SIZE", [("ra::layout_kernel(...)", calib / 1024 / 4),
                                     ("ra::layout_kernel(...)", calib / 1024),
                                     ("void ra::chunk_bwd_kv_pp_kernel<128, true>(ra::KParams)", 50.0),
                                     ("void ra::chunk_bwd_kv_pp_kernel<128, true>(ra::KParams)", 50.0),
                                     ("ra::copy2d_kernel(...)", stage / 1024 / 1.5)])
    out = tmp_path / "rec.json"
    monkeypatch.setattr(bench, "traffic_path", lambda name: str(out))
    bench.traffic_summary("wl", fdir, wdir, calib, stage)
    rec = json.load(open(out))
    k = rec["kernels"]["chunk_bwd_kv_pp_kernel"]
    assert k["fetch_bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2)
    assert k["write_bytes_per_launch"] == pytest.approx(50.0 * 1024)
    assert rec["source_hash"] == bench.source_hash()
    # the second calibration copy's factors are recorded beside the first
    assert rec["check"]["fetch_scale"] == pytest.approx(3.0)
    assert rec["check"]["write_scale"] == pytest.approx(1.5)


@pytest.mark.parametrize("window,chunk", [(0, 0), (5, 0), (0, 8), (7, 12), (1, 0)])
def test_visible_count_matches_oracle_visibility(window, chunk):
    import numpy as np
    from oracle import attn64 as O
    for q0, k0, ql, kl in [(40, 0, 16, 16), (40, 40, 16, 16), (100, 30, 20, 24), (7, 7, 9, 9)]:
        qp = np.arange(q0, q0 + ql)
        kp = np.arange(k0, k0 + kl)
        ref = int(O.visible(qp, kp, window, chunk).sum())
        assert bench.visible_count(q0, k0, ql, kl, window, chunk) == ref


def test_windowed_flops_equal_visible_pairs():
    """With a window the counted forward FLOPs are 4 d per visible pair, summed over the plan."""
    import numpy as np
    from oracle import attn64 as O
    prob = api.Problem(1, 512, 2, 1, 64, 4, "zigzag", "bf16", 0.0, 40, 0)
    for rank in range(4):
        qpos = O.rank_positions(512, 4, "zigzag", rank)
        vis = O.visible(qpos, np.arange(512), 40, 0).sum()
        assert sum(bench.counted_flops(api, prob, rank)) == 4 * 64 * vis * 2
