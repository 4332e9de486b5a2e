"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic byte counts the roofline
uses (each checked against the sum of its tensors' sizes written out term by term), and the
copy-calibrated traffic summary on synthetic counter files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_scan_bytes_is_each_tensor_once():
    b, L, d, n, es = 8, 2048, 1536, 16, 2
    x = delta = z = y = b * L * d * es
    B = C = b * L * n * es
    A = d * n * 4
    D = bias = d * 4
    last_state = b * d * n * 4
    assert bench.scan_bytes(b, L, d, n, es) == x + delta + z + y + B + C + A + D + bias + last_state == 203_272_192
    assert bench.scan_bytes(b, L, d, n, es, has_z=False) == 203_272_192 - z


def test_decode_bytes_is_state_read_and_written_once():
    b, d, n, es = 64, 5120, 16, 2
    state = 2 * b * d * n * 4
    x = delta = z = y = b * d * es
    B = C = b * n * es
    A = d * n * 4
    D = bias = d * 4
    assert bench.decode_bytes_per_step(b, d, n, es) == state + x + delta + z + y + B + C + A + D + bias == 44_937_216


def test_conv_and_ssd_bytes():
    b, L, d, k, es = 8, 2048, 1536, 4, 2
    x = y = b * L * d * es
    weight_bias = d * (k + 1) * 4
    final_state = b * d * (k - 1) * es
    assert bench.conv_bytes(b, L, d, k, es) == x + y + weight_bias + final_state == 100_767_744
    w = W.SSD_WORKLOADS["mamba2_layer_b8"]
    xzy = 3 * w.batch * w.seqlen * w.nheads * w.headdim * 2
    dt = w.batch * w.seqlen * w.nheads * 2
    BC = 2 * w.batch * w.seqlen * w.ngroups * w.dstate * 2
    params = 3 * w.nheads * 4
    final = w.batch * w.nheads * w.headdim * w.dstate * 4
    assert bench.ssd_bytes(w) == xzy + dt + BC + params + final == 429_916_928


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (kernel, value) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    scan = "void ssm::scan_chunk_kernel<true, 16, 4, 0, 32, false>(ssm::ScanArgs)"
    kib = bench.CALIB_BYTES / 1024
    # the counters read half the copy's fetched bytes and all of its written bytes; the scan's
    # median dispatch is taken
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, kib / 2), (scan, 70000.0), (scan, 80000.0),
                                                    (scan, 75000.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, kib), (scan, 50000.0), (scan, 49000.0), (scan, 51000.0)])
    rec = bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "mamba130m", out_dir=str(tmp_path))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_kib_per_launch"] == 75000.0 and rec["write_kib_per_launch"] == 50000.0
    assert rec["hbm_bytes_per_launch"] == pytest.approx(75000 * 1024 * 2 + 50000 * 1024)
    assert rec["alg_bytes_per_launch"] == 203_272_192
    assert rec["source_hash"] == bench.source_hash("scan")
    assert json.load(open(tmp_path / "traffic_mamba130m.json")) == rec


def test_method_slots_term_by_term():
    """The VALU co-bound's method work: 6 slots per (t,d,n) update (dt*A, v_exp_f32 at half rate,
    B*(dt x), the state FMA, the read-out FMA) and 14 per (t,d) (softplus and SiLU)."""
    elems, n = 8 * 2048 * 1536, 16
    per_update = 1 + 2 + 1 + 1 + 1
    assert bench.SLOTS_PER_UPDATE == per_update
    assert bench.method_slots(elems, n) == elems * n * per_update + elems * bench.SLOTS_PER_TD
    assert abs(bench.method_slots(elems, n) / (elems * n) - 6.875) < 1e-12


def test_valu_ceiling_against_the_hbm_target():
    """The bench line's target block: at 100% fp32 issue with zero overhead the 130M-shaped scan
    takes method_slots / 39.3 T slots/s = 70.4 us, i.e. its 203,272,192 algorithmic bytes at 36% of
    8 TB/s, so the 60% target lies above what this arithmetic allows without packed fp32."""
    elems, n = 8 * 2048 * 1536, 16
    floor_s = bench.method_slots(elems, n) / bench.VALU_LANE_SLOTS
    assert abs(floor_s * 1e6 - 70.4) < 0.05
    ceiling = bench.scan_bytes(8, 2048, 1536, 16, 2) / floor_s / 1e9 / bench.HBM_PEAK_GBPS
    assert 0.36 < ceiling < 0.362
    assert ceiling < bench.HBM_TARGET_FRAC
