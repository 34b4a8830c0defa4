"""Host-side checks of bench.py: the algorithmic byte counts that every
roofline fraction divides by (written out here from the shapes), the scaling
of the counter summary by a copy kernel, and the refusal of more than one GPU.
Nothing here touches a GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ssd_inputs as si  # noqa: E402


def test_scan_bytes_at_the_2p7b_shape():
    w = si.WORKLOADS["m2_2p7b"]
    B, L, H, P, N = 4, 4096, 80, 64, 128
    xy = 2 * B * L * H * P * 2
    dt = B * L * H * 4
    bc = 2 * B * L * N * 2
    ad = 2 * H * 4
    states = 2 * B * H * P * N * 4          # initial state in, final state out
    assert bench.scan_algorithmic(w)[0] == xy + dt + bc + ad + states == 370_147_968


def test_scan_flops_count_the_decomposition_that_runs():
    # the per-sequence scan walks 64-token sub-blocks whatever the chunk size,
    # so the flops the bench divides by are those of 64-token blocks
    w = si.WORKLOADS["m2_2p7b"]
    assert bench.per_sequence_scan(w) and bench.per_sequence_scan(si.WORKLOADS["long_n256"])
    assert not bench.per_sequence_scan(si.WORKLOADS["tiny_fp32"])
    B, L, H, P, N, q = 4, 4096, 80, 64, 128, 64
    nc, tri = L // q, q * (q + 1) // 2
    flops = (2 * B * nc * tri * N + 2 * B * nc * H * tri * P + 4 * B * L * H * P * N
             + 2 * B * nc * H * P * N + 2 * B * L * H * P)
    assert bench.scan_algorithmic(w, 64)[1] == flops
    assert bench.scan_algorithmic(w)[1] > flops          # blocks of 256: larger quadratic terms


def test_backward_and_block_bytes_at_the_2p7b_shape():
    w = si.WORKLOADS["m2_2p7b"]
    B, L, H, P, N = 4, 4096, 80, 64, 128
    bwd = (3 * B * L * H * P * 2 + 2 * B * L * H * 4 + 4 * B * L * N * 2 + 4 * H * 4
           + B * H * P * N * 4 + 2 * B * H * P * N * 4)
    assert bench.bwd_algorithmic(w) == bwd == 562_038_016
    T, HP, GN = B * L, H * P, N
    pro = T * (HP + 2 * GN + H) * 2 + T * (HP + 2 * GN) * 2 + T * H * 4
    assert bench.block_algorithmic(w) == (pro, 3 * T * HP * 2) == (360_185_856, 503_316_480)


def _counter_csv(folder, counter, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, (name, v) in enumerate(rows):
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_mb = 512.0
    # the copy reads and writes 512e6 bytes; its counters read 250,000 and 500,000 KiB
    _counter_csv(tmp_path / "cf", "FETCH_SIZE", [("stream_copy(unsigned int const*)", 250_000.0)])
    _counter_csv(tmp_path / "cw", "WRITE_SIZE", [("stream_copy(unsigned int const*)", 500_000.0)])
    # two dispatches of each scan kernel, one of a backward kernel
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [("void pipe_kernel<128, false>(Args)", 100.0),
                                                ("void pipe_kernel<128, false>(Args)", 300.0),
                                                ("void prep_kernel<128, false>(Args, int)", 10.0),
                                                ("void chunk_grad<128>(BwdArgs)", 1000.0),
                                                ("void step_kernel<bf16, 64, 128>(float*)", 700.0)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [("void pipe_kernel<128, false>(Args)", 50.0),
                                                ("void pipe_kernel<128, false>(Args)", 50.0),
                                                ("void prep_kernel<128, false>(Args, int)", 5.0),
                                                ("void chunk_grad<128>(BwdArgs)", 400.0),
                                                ("void step_kernel<bf16, 64, 128>(float*)", 600.0)])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"), copy_mb)
    t = json.load(open(tmp_path / "traffic.json"))
    ff, fw = 512e6 / 250_000, 512e6 / 500_000
    assert t["fetch_scale_bytes_per_kib"] == pytest.approx(ff) and t["write_scale_bytes_per_kib"] == pytest.approx(fw)
    pipe = t["kernels"]["pipe_kernel"]
    assert pipe["fetch_kib"] == pytest.approx(200.0) and pipe["write_kib"] == pytest.approx(50.0)   # per-dispatch means
    assert t["bytes_per_launch"] == pytest.approx(200.0 * ff + 50.0 * fw + 10.0 * ff + 5.0 * fw)
    assert t["bwd_bytes_per_call"] == pytest.approx(1000.0 * ff + 400.0 * fw)
    assert t["step_bytes_per_call"] == pytest.approx(700.0 * ff + 600.0 * fw)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_inputs_are_made_once_and_shared():
    # the bench makes every input before its first measurement; later calls
    # find them instead of drawing them again (on the host here, a small shape)
    import torch
    w = si.WORKLOADS["tiny_fp32"]
    dev = torch.device("cpu")
    a = bench.make_device_sets(w, 2, dev)
    assert bench.make_device_sets(w, 2, dev) is a
    bench.add_grad_inputs(w, a, dev)
    dy = [s["dy"] for s in a]
    bench.add_grad_inputs(w, a, dev)
    assert all(s["dy"] is d for s, d in zip(a, dy))
    n = bench.add_varlen_inputs(w, a, dev)
    assert n == bench.add_varlen_inputs(w, a, dev) and all(k >= 1 for k in n)
    assert all(s["yv"] is not s["y"] and s["yv"] is not s["x"] for s in a)
    st, ins, ys = bench.step_inputs(2, 2, 16, 16, 1, dev)
    assert bench.step_inputs(2, 2, 16, 16, 1, dev)[0] is st and len(ins) == len(ys) == 4
