#!/usr/bin/env python3
"""Benchmark of the SSD chunk scan on one MI355X.

One step = one ssd_chunk_scan_fwd call over the Mamba-2 2.7B-layer workload
(B=4, L=4096, H=80, P=64, N=128, G=1, chunk 256, bf16 x/Bm/Cm/y, fp32 dt/A/D
and states, random initial state).  Inputs are resident in HBM before the
timed region; three input/output sets are rotated so that no step finds the
previous step's data in the 256 MB Infinity Cache.  The decode step
(ssd_step, B=256, H=80, P=64, N=128) is timed the same way and reported in
its own object.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Measurement helpers (used to produce the files under profiles/):
  python bench.py --calibrate-copy MB [--steps K]
      only a plain device copy of MB megabytes, K times (the reference kernel
      for scaling the FETCH_SIZE / WRITE_SIZE counters);
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR --copy-mb MB
      turns four `rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE` output folders into
      profiles/traffic_m2_2p7b.json (HBM bytes per scan launch);
  python bench.py --summarize-mfma DIR [--cus 256] [--xcds 8]
      per-kernel matrix-core utilisation from a `rocprofv3 --pmc
      SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE` output folder.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_m2_2p7b.json")
WORKLOAD_NAMES = {"m2_2p7b": "mamba2_2.7b_layer_ssd_chunk_scan", "m2_130m": "mamba2_130m_layer_ssd_chunk_scan",
                  "tiny_fp32": "tiny_fp32_ssd_chunk_scan", "long_n128": "long_sequence_n128_ssd_chunk_scan",
                  "long_n256": "long_sequence_n256_ssd_chunk_scan",
                  "m2_2p7b_p128": "mamba2_2.7b_layer_head_dim_128_ssd_chunk_scan"}
# what each workload is, for the metric string of its line
WORKLOAD_DESC = {"m2_2p7b": "Mamba-2 2.7B layer shape", "m2_130m": "Mamba-2 130M layer shape",
                 "tiny_fp32": "tiny fp32 shape", "long_n128": "long-sequence shape, N=128",
                 "long_n256": "long-sequence shape, N=256",
                 "m2_2p7b_p128": "Mamba-2 2.7B layer channels as 40 heads of 128"}
HEADLINE_METRIC = "SSD chunk-scan fwd tokens/s at Mamba-2 2.7B layer shape; % of roofline"
# the sources whose kernels run in one scan launch at this workload
SCAN_SOURCES = ["pipe_scan.hip", "tile_ops.h", "mfma_scan.hip", "api.hip", "common.h"]
# and in one backward call, and one decode step
BWD_SOURCES = ["bwd_scan.hip", "api.hip", "common.h"]
STEP_SOURCES = ["step.hip", "api.hip", "common.h"]
BWD_KERNELS = ("state_scans", "chunk_grad", "reduce_head")


def scan_sources_digest(files=SCAN_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "selective_state_space_chunk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def per_sequence_scan(w):
    """Whether the library's default path for this workload is the
    per-sequence scan, which walks 64-token sub-blocks whatever the chunk."""
    return w.dtype == "bf16" and w.P in (64, 128) and w.N in (64, 128, 256)


def scan_algorithmic(w, q=None):
    """Bytes every input read once + outputs written once; flops of the block
    decomposition into blocks of q tokens (default: the chunk size) with the
    causal halves of the quadratic terms."""
    B, L, H, P, N, G = w.B, w.L, w.H, w.P, w.N, w.G
    Q = q or w.chunk
    e = 2 if w.dtype == "bf16" else 4
    nc = -(-L // Q)
    byts = (2 * B * L * H * P * e          # x in, y out
            + B * L * H * 4                # dt
            + 2 * B * L * G * N * e        # Bm, Cm
            + 2 * H * 4                    # A, D
            + (B * H * P * N * 4 if w.init else 0)   # initial state
            + B * H * P * N * 4)           # final state
    tri = Q * (Q + 1) // 2
    flops = (2 * B * nc * G * tri * N      # Cm Bm^T, causal
             + 2 * B * nc * H * tri * P    # masked product with x
             + 2 * B * L * H * P * N       # block states
             + 2 * B * L * H * P * N       # state -> output
             + 2 * B * nc * H * P * N      # state pass
             + 2 * B * L * H * P)          # D skip
    return byts, flops


def bwd_algorithmic(w):
    """Bytes of the backward read or written once: x, dy, dt, Bm, Cm, the
    initial state and dfinal in; dx, ddt, dBm, dCm, dA, dD, dinit out."""
    B, L, H, P, N, G = w.B, w.L, w.H, w.P, w.N, w.G
    e = 2 if w.dtype == "bf16" else 4
    return (3 * B * L * H * P * e          # x, dy in; dx out
            + 2 * B * L * H * 4            # dt in, ddt out
            + 4 * B * L * G * N * e        # Bm, Cm in; dBm, dCm out
            + 4 * H * 4                    # A, D in; dA, dD out
            + (B * H * P * N * 4 if w.init else 0)   # initial state
            + 2 * B * H * P * N * 4)       # dfinal in, dinit out


def step_algorithmic(B, H, P, N, G, e=2):
    byts = (2 * B * H * P * N * 4          # state read + write
            + 2 * B * H * P * e            # x in, y out
            + B * H * 4                    # dt
            + 2 * B * G * N * e            # Bm, Cm
            + 2 * H * 4)
    return byts


_SETS = {}


def make_device_sets(w, nsets, device):
    """Seeded input sets of workload w, resident on the device; made once per
    (workload, count, device) and shared by the measurements that use them
    (each writes only outputs of its own)."""
    import torch
    import ssd_inputs as si
    key = (w.name, nsets, str(device))
    if key in _SETS:
        return _SETS[key]
    sets = []
    for k in range(nsets):
        d = si.make_scan_inputs(w.B, w.L, w.H, w.P, w.N, w.G, dtype=w.dtype, init=w.init,
                                seed=w.seed + 100 * k)
        td = {}
        for name, v in d.items():
            if v is None:
                td[name] = None
            elif name in ("x", "Bm", "Cm"):
                td[name] = torch.from_numpy(v).to(device=device, dtype=io_dtype(w))
            else:
                td[name] = torch.from_numpy(v).to(device=device, dtype=torch.float32)
        td["y"] = torch.empty_like(td["x"])
        td["final"] = torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device=device)
        sets.append(td)
    _SETS[key] = sets
    return sets


def add_grad_inputs(w, sets, device):
    """dy and dfinal of each input set (seeded), for the backward."""
    import torch
    import ssd_inputs as si
    for k, s in enumerate(sets):
        if "dy" not in s:
            g = si.make_grad_inputs(w.B, w.L, w.H, w.P, w.N, dtype=w.dtype, seed=w.seed + 100 * k + 7)
            s["dy"] = torch.from_numpy(g["dy"]).to(device=device, dtype=io_dtype(w))
            s["dfinal"] = torch.from_numpy(g["dfinal"]).to(device=device)


def add_varlen_inputs(w, sets, device):
    """Document boundaries of each input set: rows packed with documents of
    log-normal length (median VARLEN_MEAN_LEN tokens, the last one cut at
    the row's end); returns the number of documents per set."""
    import torch
    import ssd_inputs as si
    for k, s in enumerate(sets):
        if "seq" not in s:
            seq = si.make_seq_idx(w.B, w.L, mean_len=VARLEN_MEAN_LEN, seed=w.seed + 100 * k + 9)
            s["nseq"] = int(sum(seq[b, -1] + 1 for b in range(w.B)))
            s["seq"] = torch.from_numpy(seq).to(device)
            s["yv"] = torch.empty_like(s["x"])
            s["fv"] = torch.empty((w.B, w.H, w.P, w.N), dtype=torch.float32, device=device)
    return [s["nseq"] for s in sets]


_STEP = {}


def step_inputs(B, H, P, N, G, device):
    """The decode state and four tokens' inputs (seeded), resident on the
    device; made once per shape."""
    import torch
    import ssd_inputs as si
    key = (B, H, P, N, G, str(device))
    if key not in _STEP:
        st = torch.from_numpy(si.make_step_state(B, H, P, N, seed=si.SEED_BASE + 4)).to(device)
        ins = []
        for t in range(4):
            s = si.make_step_inputs(B, H, P, N, G, step=t, dtype="bf16", seed=si.SEED_BASE + 4)
            ins.append({k: torch.from_numpy(v).to(device, dtype=torch.bfloat16 if k in ("x", "Bm", "Cm")
                                                   else torch.float32) for k, v in s.items()})
        _STEP[key] = (st, ins, [torch.empty_like(i["x"]) for i in ins])
    return _STEP[key]


def io_dtype(w):
    import torch
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def time_scan(w, steps, warmup, device, algo="auto"):
    import torch
    import selective_state_space_chunk_amd as ssd
    sets = make_device_sets(w, 3, device)
    nbytes = ssd.ssd_chunk_scan_workspace_size(w.B, w.L, w.H, w.P, w.G, w.N, w.chunk, io_dtype(w), algo)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def run(k):
        s = sets[k % len(sets)]
        ssd.ssd_chunk_scan_fwd(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], s["D"], s["init"], w.chunk,
                               y=s["y"], final_state=s["final"], workspace_tensor=ws, algo=algo)

    for k in range(warmup):
        run(k)
    torch.cuda.synchronize(device)
    # the timed steps: back to back, the wall clock around them
    t0 = time.perf_counter()
    for k in range(steps):
        run(k)
    torch.cuda.synchronize(device)
    wall = time.perf_counter() - t0
    # then the same number of calls again, each between two events on the
    # stream the library launches on (the current stream): the kernels' own
    # time, without the gaps the event markers add between calls
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record()
        run(k)
        ends[k].record()
    torch.cuda.synchronize(device)
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))   # ms
    return wall, per


def time_step(B, H, P, N, G, steps, warmup, device):
    import torch
    import selective_state_space_chunk_amd as ssd
    st, ins, ys = step_inputs(B, H, P, N, G, device)
    for k in range(warmup):
        i = ins[k % 4]
        ssd.ssd_step(st, i["x"], i["dt"], i["A"], i["Bm"], i["Cm"], i["D"], y=ys[k % 4])
    torch.cuda.synchronize(device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        i = ins[k % 4]
        starts[k].record()
        ssd.ssd_step(st, i["x"], i["dt"], i["A"], i["Bm"], i["Cm"], i["D"], y=ys[k % 4])
        ends[k].record()
    torch.cuda.synchronize(device)
    return sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


def time_backward(w, steps, warmup, device):
    """Per-call event times (ms) of ssd_chunk_scan_bwd over rotating input sets."""
    import torch
    import selective_state_space_chunk_amd as ssd
    import ssd_inputs as si
    sets = make_device_sets(w, 3, device)
    add_grad_inputs(w, sets, device)
    nbytes = ssd.ssd_chunk_scan_bwd_workspace_size(w.B, w.L, w.H, w.P, w.G, w.N, w.chunk, io_dtype(w))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def run(k):
        s = sets[k % len(sets)]
        ssd.ssd_chunk_scan_bwd(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], s["D"], s["init"], s["dy"],
                               s["dfinal"], w.chunk, workspace_tensor=ws)

    for k in range(warmup):
        run(k)
    torch.cuda.synchronize(device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record()
        run(k)
        ends[k].record()
    torch.cuda.synchronize(device)
    return sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


VARLEN_MEAN_LEN = 512.0
CONV_WIDTH = 4


def block_algorithmic(w):
    """Bytes of the block prologue (the x, Bm, Cm and dt slices of the
    projection output read once; x, Bm, Cm and dt written once) and of the
    gated norm (y and z read once, the output written once)."""
    bl, hp, gn = w.B * w.L, w.H * w.P, w.G * w.N
    pro = bl * (hp + 2 * gn + w.H) * 2 + bl * (hp + 2 * gn) * 2 + bl * w.H * 4
    norm = 3 * bl * hp * 2
    return pro, norm


def time_block(w, steps, warmup, device):
    """Per-call event times (ms) of ssd_block_prologue and ssd_gated_norm at the
    workload's shape, over two rotating sets of projection outputs and scan
    outputs drawn on the device from a seeded generator (N(0, 1), bfloat16)."""
    import torch
    import selective_state_space_chunk_amd as ssd
    import ssd_inputs as si
    small = si.make_block_inputs(1, 1, w.H, w.P, w.G, w.N, CONV_WIDTH, seed=w.seed + 11)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 12)
    row = 2 * w.H * w.P + 2 * w.G * w.N + w.H
    sets = [{"zx": torch.randn((w.B, w.L, row), generator=gen, device=device).to(torch.bfloat16),
             "y": torch.randn((w.B, w.L, w.H, w.P), generator=gen, device=device).to(torch.bfloat16)}
            for _ in range(2)]
    cw, cb, db = (torch.from_numpy(small[k]).to(device) for k in ("conv_w", "conv_b", "dt_bias"))
    nw, nb = (torch.from_numpy(small[k]).to(device) for k in ("norm_w", "norm_b"))
    outs = [ssd.ssd_block_prologue(s["zx"], cw, cb, db, w.H, w.P, w.G, w.N) for s in sets]
    nout = torch.empty_like(sets[0]["y"])

    def run_pro(k):
        s = sets[k % 2]
        ssd.ssd_block_prologue(s["zx"], cw, cb, db, w.H, w.P, w.G, w.N)

    def run_norm(k):
        ssd.ssd_gated_norm(sets[k % 2]["y"], outs[k % 2]["z"], nw, nb, 1, 1e-5, True, out=nout)

    res = []
    for fn in (run_pro, run_norm):
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize(device)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for k in range(steps):
            starts[k].record()
            fn(k)
            ends[k].record()
        torch.cuda.synchronize(device)
        res.append(sorted(a.elapsed_time(b) for a, b in zip(starts, ends)))
    return res


def time_varlen(w, steps, warmup, device):
    """Per-call event times (ms) of ssd_chunk_scan_fwd_varlen over rotating
    input sets, each row packed with documents of log-normal length (median
    512 tokens, the last one cut at the row's end)."""
    import torch
    import selective_state_space_chunk_amd as ssd
    import ssd_inputs as si
    sets = make_device_sets(w, 3, device)
    nseq = add_varlen_inputs(w, sets, device)
    nbytes = ssd.ssd_chunk_scan_varlen_workspace_size(w.B, w.L, w.H, w.P, w.G, w.N, w.chunk, io_dtype(w))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)

    def run(k):
        s = sets[k % len(sets)]
        ssd.ssd_chunk_scan_fwd_varlen(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], s["D"], s["seq"], s["init"],
                                      w.chunk, y=s["yv"], final_state=s["fv"], workspace_tensor=ws)

    for k in range(warmup):
        run(k)
    torch.cuda.synchronize(device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record()
        run(k)
        ends[k].record()
    torch.cuda.synchronize(device)
    return sorted(s.elapsed_time(e) for s, e in zip(starts, ends)), nseq


# Mamba-1 2.8B layer: d_inner 5120 channels, N = 16 states, the same 4 x 4096 tokens
S6_SHAPE = {"batch": 4, "seq_len": 4096, "channels": 5120, "state": 16, "groups": 1}
# vector-ALU issue slots per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (non-packed fp32)
VALU_LANE_SLOTS = 256 * 4 * 16 * 2.4e9
# slots one state update needs at least: one exp2 (a quarter-rate transcendental, 4 slots)
# and three multiply-adds (dt A, the input term, the output sum)
S6_SLOTS_PER_UPDATE = 7


def time_s6(steps, warmup, device):
    """Per-call event times (ms) of ssd_selective_scan (zero-order hold) over two
    rotating input sets drawn on the device from a seeded generator."""
    import torch
    import selective_state_space_chunk_amd as ssd
    B, L, Dch, N = (S6_SHAPE[k] for k in ("batch", "seq_len", "channels", "state"))
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED_S6)
    sets = []
    for _ in range(2):
        sets.append({"x": torch.randn((B, L, Dch), generator=gen, device=device).to(torch.bfloat16),
                     "dt": torch.nn.functional.softplus(torch.randn((B, L, Dch), generator=gen, device=device) - 1.0
                                                        ).to(torch.bfloat16),
                     "Bm": torch.randn((B, L, 1, N), generator=gen, device=device).to(torch.bfloat16),
                     "Cm": torch.randn((B, L, 1, N), generator=gen, device=device).to(torch.bfloat16)})
    A = -torch.exp(torch.rand((Dch, N), generator=gen, device=device) * 2.5 - 1.0)
    D = torch.randn((Dch,), generator=gen, device=device)
    init = torch.randn((B, Dch, N), generator=gen, device=device) * 0.3

    def run(k):
        s = sets[k % 2]
        ssd.ssd_selective_scan(s["x"], s["dt"], A, s["Bm"], s["Cm"], D, init, zoh=True)

    for k in range(warmup):
        run(k)
    torch.cuda.synchronize(device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for k in range(steps):
        starts[k].record()
        run(k)
        ends[k].record()
    torch.cuda.synchronize(device)
    return sorted(a.elapsed_time(b) for a, b in zip(starts, ends))


SEED_S6 = 20240531


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle (token-by-token recurrence, OpenMP over (batch, head)
    sequences) on a bounded sample of the same workload: whole sequences of
    some of the B*H (batch, head) pairs, spread over all batch rows, scaled to
    tokens/s of the full layer (a token is all H heads of one position)."""
    import oracle
    import ssd_inputs as si
    threads = oracle.num_threads()
    f = si.as_f64(si.workload_scan_inputs(w))
    chains = w.B * w.H
    order = [(k % w.B) * w.H + (k // w.B) % w.H for k in range(chains)]   # batch rows interleaved
    n = max(1, min(chains, threads))
    t0 = time.perf_counter()
    oracle.recurrence(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], bh=order[:n])
    probe = time.perf_counter() - t0
    # grow the sample toward the budget in whole rounds of `threads` sequences;
    # when the whole workload takes less, run it repeatedly until the budget
    rounds = max(1, int(budget_s / max(probe, 1e-3)))
    n = max(1, min(chains, n * rounds))
    reps, el = 0, 0.0
    while reps == 0 or el < 0.7 * budget_s:
        t0 = time.perf_counter()
        oracle.recurrence(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], bh=order[:n])
        el += time.perf_counter() - t0
        reps += 1
    return {"value": reps * n * w.L / el / w.H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 token-by-token recurrence over {n} of the {chains} (batch, head) "
                      f"sequences of L={w.L} tokens, {reps} run(s), {el:.1f} s on {threads} threads; "
                      f"tokens/s = runs*sequences*L/s / H"}


def copy_bandwidth(device, mb=512, reps=10, warm=200):
    """Measured bandwidth (GB/s, bytes read + written) of the library's own
    streaming copy (ssd_stream_copy) of `mb` megabytes, median of `reps`
    event-timed launches after `warm` untimed ones (~30 ms, the clock ramp
    of an idle device): what a kernel with no arithmetic moves here, the
    practical ceiling the achieved bandwidths are also reported against."""
    import torch
    import selective_state_space_chunk_amd as ssd
    n = int(mb * 1e6) // 16 * 4
    src = torch.ones(n, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(warm):
        ssd.ssd_stream_copy(dst, src)
    torch.cuda.synchronize(device)
    times = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        ssd.ssd_stream_copy(dst, src)
        e.record()
        torch.cuda.synchronize(device)
        times.append(s.elapsed_time(e))
    times.sort()
    return 2 * n * 4 / (times[len(times) // 2] * 1e-3) / 1e9


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def traffic_file(workload="m2_2p7b"):
    """The counter summary of a scan workload (the headline's holds the
    backward, decode and block-step figures too)."""
    if workload == "m2_2p7b":
        return TRAFFIC_FILE
    return os.path.join(os.path.dirname(TRAFFIC_FILE), f"traffic_{workload}.json")


def scan_traffic(workload="m2_2p7b"):
    """HBM bytes per scan launch from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(traffic_file(workload)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != scan_sources_digest():
        return None
    return t.get("bytes_per_launch")


def step_traffic():
    """HBM bytes per decode step from the same summary, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("step_sources_sha256") != scan_sources_digest(STEP_SOURCES):
        return None
    return t.get("step_bytes_per_call")


def bwd_traffic():
    """HBM bytes per backward call from the same summary, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("bwd_sources_sha256") != scan_sources_digest(BWD_SOURCES):
        return None
    return t.get("bwd_bytes_per_call")


def calibrate_copy(mb, steps):
    """Only the library's streaming copy (stream_copy) of `mb` megabytes,
    `steps` times: the reference kernel for scaling the counters."""
    import torch
    import selective_state_space_chunk_amd as ssd
    n = int(mb * 1e6) // 16 * 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        ssd.ssd_stream_copy(dst, src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": steps}))


def _pmc_kib(folder, counter, match):
    """Mean per-dispatch value (KiB) of `counter` over kernels whose name
    contains `match`, from a rocprofv3 --pmc csv folder."""
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter and match in row["Kernel_Name"]:
                    vals.setdefault(row["Dispatch_Id"], 0.0)
                    vals[row["Dispatch_Id"]] += float(row["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} rows for kernels matching {match!r} in {folder}")
    return sum(vals.values()) / len(vals), len(vals)


def summarize_mfma(folder, cus, xcds):
    """Per-kernel matrix-core utilisation from a rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: busy cycles (summed over
    all SIMDs: 16 per 16x16x32 bf16 instruction) over (active cycles x compute
    units x 4 SIMDs), averaged over dispatches.  GRBM_GUI_ACTIVE comes summed
    over the XCDs, so it is divided by their number."""
    rows = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                d = rows.setdefault((row["Kernel_Name"], row["Dispatch_Id"]), {})
                d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    per = {}
    for (name, _), d in rows.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" in d and d.get("GRBM_GUI_ACTIVE"):
            active = d["GRBM_GUI_ACTIVE"] / xcds
            per.setdefault(name, []).append(d["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * cus * 4))
    out = {n: {"dispatches": len(v), "mfma_util": sum(v) / len(v)} for n, v in per.items()}
    print(json.dumps(out, indent=1))


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mb, workload="m2_2p7b"):
    copy_bytes = int(copy_mb * 1e6) // 4 * 4
    cf, _ = _pmc_kib(copy_fetch_dir, "FETCH_SIZE", "copy")
    cw, _ = _pmc_kib(copy_write_dir, "WRITE_SIZE", "copy")
    f_fetch, f_write = copy_bytes / cf, copy_bytes / cw      # bytes per counted KiB
    out = {"workload": workload, "sources_sha256": scan_sources_digest(),
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale_bytes_per_kib": f_fetch, "write_scale_bytes_per_kib": f_write, "kernels": {}}
    total = 0.0
    for name in ("pipe_kernel", "prep_kernel"):
        try:
            fk, nf = _pmc_kib(fetch_dir, "FETCH_SIZE", name)
            wk, nw = _pmc_kib(write_dir, "WRITE_SIZE", name)
        except SystemExit:
            continue
        b = fk * f_fetch + wk * f_write
        out["kernels"][name] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                                "read_bytes": fk * f_fetch, "write_bytes": wk * f_write}
        total += b
    out["bytes_per_launch"] = total
    out["bwd_sources_sha256"] = scan_sources_digest(BWD_SOURCES)
    out["bwd_kernels"] = {}
    btotal = 0.0
    for name in BWD_KERNELS:
        try:
            fk, nf = _pmc_kib(fetch_dir, "FETCH_SIZE", name)
            wk, nw = _pmc_kib(write_dir, "WRITE_SIZE", name)
        except SystemExit:
            continue
        out["bwd_kernels"][name] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                                    "read_bytes": fk * f_fetch, "write_bytes": wk * f_write}
        btotal += fk * f_fetch + wk * f_write
    out["bwd_bytes_per_call"] = btotal if out["bwd_kernels"] else None
    # the staged form (an explicit choice, not the headline call), per kernel
    out["staged_kernels"] = {}
    for name, match in (("gram_kernel", "gram_kernel"),
                        ("scan_mfma<kState>", "scan_mfmaILi128ELi256ELi0E"),      # N 128, chunk 256, mode 0
                        ("scan_mfma<kOutput>", "scan_mfmaILi128ELi256ELi1E"),     # mode 1
                        ("state_pass_kernel", "state_pass_kernel")):
        try:
            fk, nf = _pmc_kib(fetch_dir, "FETCH_SIZE", match)
            wk, nw = _pmc_kib(write_dir, "WRITE_SIZE", match)
        except SystemExit:
            continue
        out["staged_kernels"][name] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                                       "read_bytes": fk * f_fetch, "write_bytes": wk * f_write}
    out["step_sources_sha256"] = scan_sources_digest(STEP_SOURCES)
    out["step_kernels"] = {}
    try:
        fk, nf = _pmc_kib(fetch_dir, "FETCH_SIZE", "step_kernel")
        wk, nw = _pmc_kib(write_dir, "WRITE_SIZE", "step_kernel")
        out["step_kernels"]["step_kernel"] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                                              "read_bytes": fk * f_fetch, "write_bytes": wk * f_write}
        out["step_bytes_per_call"] = fk * f_fetch + wk * f_write
    except SystemExit:
        out["step_bytes_per_call"] = None
    out["block_kernels"] = {}
    for name in ("prologue_kernel", "gated_norm_kernel"):
        try:
            fk, nf = _pmc_kib(fetch_dir, "FETCH_SIZE", name)
            wk, nw = _pmc_kib(write_dir, "WRITE_SIZE", name)
        except SystemExit:
            continue
        out["block_kernels"][name] = {"fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw],
                                      "read_bytes": fk * f_fetch, "write_bytes": wk * f_write}
    path = traffic_file(workload)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-block", action="store_true")
    ap.add_argument("--no-s6", action="store_true")
    ap.add_argument("--no-staged", action="store_true")
    ap.add_argument("--calibrate-copy", type=float, default=None, metavar="MB")
    ap.add_argument("--summarize-pmc", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--copy-mb", type=float, default=512.0)
    ap.add_argument("--summarize-mfma", default=None, metavar="DIR")
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--xcds", type=int, default=8)
    ap.add_argument("--workload", default="m2_2p7b",
                    help="scan workload to time (m2_2p7b is the headline; tiny_fp32, m2_130m, long_n128, "
                         "long_n256 and m2_2p7b_p128 are the other scan shapes)")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.copy_mb, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.cus, args.xcds)
        return
    if args.calibrate_copy is not None:
        calibrate_copy(args.calibrate_copy, args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the scan has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import ssd_inputs as si
    device = torch.device("cuda:0")
    if args.workload not in si.WORKLOADS or si.WORKLOADS[args.workload].L < 2:
        raise SystemExit(f"unknown scan workload {args.workload!r}")
    w = si.WORKLOADS[args.workload]
    headline = args.workload == "m2_2p7b"
    # the flops of the decomposition the kernels run: 64-token sub-blocks on
    # the per-sequence scan, blocks of the chunk size otherwise
    block = 64 if per_sequence_scan(w) else w.chunk
    byts, flops = scan_algorithmic(w, block)
    tokens = w.B * w.L
    do_backward = not args.no_backward and (headline or (w.P == 128 and w.N <= 128 and w.dtype == "bf16"))
    # Every input is made first and kept resident; the measurements then run
    # back to back with no host work between them, the headline call last.
    # After an idle spell the device's clocks ramp up over the first ~200
    # calls (~30 ms) of sustained load (the headline call takes ~230 us cold
    # and ~146 us in steady state), so a call timed a few calls after the
    # host-side setup would measure the ramp rather than the kernel.
    make_device_sets(w, 3, device)
    if not args.no_decode:
        step_inputs(256, 80, 64, 128, 1, device)
    if do_backward:
        add_grad_inputs(w, make_device_sets(w, 3, device), device)
    if not args.no_varlen and headline:
        add_varlen_inputs(w, make_device_sets(w, 3, device), device)
    torch.cuda.synchronize(device)
    extra = {}
    copy_gbs = copy_bandwidth(device)
    if not args.no_decode:
        B, H, P, N, G = 256, 80, 64, 128, 1
        sp = time_step(B, H, P, N, G, max(20, args.steps // 2), 5, device)
        smean = sum(sp) / len(sp)
        sb = step_algorithmic(B, H, P, N, G)
        extra["decode"] = {"workload": "mamba2_2.7b_layer_ssd_step", "batch": B, "heads": H,
                           "head_dim": P, "state": N, "us_per_step": smean * 1000.0,
                           "tokens_per_s": B / (smean * 1e-3), "kernel": f"step_kernel<bf16, {P}, {N}>",
                           "roofline": {"bound": "hbm", "achieved": sb / (smean * 1e-3) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": sb / (smean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "frac_of_copy": sb / (smean * 1e-3) / 1e9 / copy_gbs,
                                        "traffic": step_traffic(), "algorithmic_bytes": sb}}
    if do_backward:
        # the backward at the layer shape, and at its head-dim-128 form
        bp = time_backward(w, max(10, args.steps // 5), 3, device)
        bmean = sum(bp) / len(bp)
        bb = bwd_algorithmic(w)
        extra["backward"] = {"workload": WORKLOAD_NAMES.get(w.name, w.name) + "_backward",
                             "us_per_call": bmean * 1000.0, "us_median": bp[len(bp) // 2] * 1000.0,
                             "tokens_per_s": tokens / (bmean * 1e-3),
                             "kernels": f"state_scans<{w.N}> (forward and adjoint states) + chunk_grad<{w.N}> + "
                                        "reduce_head",
                             "roofline": {"bound": "hbm", "achieved": bb / (bmean * 1e-3) / 1e9,
                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": bb / (bmean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                          "traffic": bwd_traffic() if headline else None,
                                          "algorithmic_bytes": bb}}
    if not args.no_block and headline:
        tp, tn = time_block(w, max(10, args.steps // 2), 3, device)
        pb, nb = block_algorithmic(w)

        def leg(ts, nbytes, kernel):
            m = sum(ts) / len(ts)
            return {"kernel": kernel, "us_per_call": m * 1000.0, "us_median": ts[len(ts) // 2] * 1000.0,
                    "roofline": {"bound": "hbm", "achieved": nbytes / (m * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                 "unit": "GB/s", "frac": nbytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                 "algorithmic_bytes": nbytes}}
        extra["block"] = {"workload": WORKLOAD_NAMES.get(w.name, w.name).replace("_ssd_chunk_scan", "_block_steps"),
                          "conv_width": CONV_WIDTH, "norm": "group norm, 1 group, eps 1e-5",
                          "prologue": leg(tp, pb, f"prologue_kernel<{CONV_WIDTH}>"),
                          "gated_norm": leg(tn, nb, "gated_norm_kernel")}
    if not args.no_s6 and headline:
        ts = time_s6(max(10, args.steps // 2), 3, device)
        m = sum(ts) / len(ts)
        sh = S6_SHAPE
        toks = sh["batch"] * sh["seq_len"]
        updates = toks * sh["channels"] * sh["state"]
        peak = VALU_LANE_SLOTS / S6_SLOTS_PER_UPDATE
        nbytes = 3 * toks * sh["channels"] * 2 + 2 * toks * sh["state"] * 2 + 2 * sh["batch"] * sh["channels"] * sh["state"] * 4
        extra["s6"] = {"workload": "mamba1_2.8b_layer_selective_scan", "config": dict(sh, discretisation="zero-order hold"),
                       "kernel": "s6_lane_kernel<16, true>", "us_per_call": m * 1000.0, "us_median": ts[len(ts) // 2] * 1000.0,
                       "tokens_per_s": toks / (m * 1e-3),
                       "roofline": {"bound": "alu", "achieved": updates / (m * 1e-3) / 1e12, "peak": peak / 1e12,
                                    "unit": "T state updates/s", "frac": updates / (m * 1e-3) / peak,
                                    "hbm_gbs": nbytes / (m * 1e-3) / 1e9, "algorithmic_bytes": nbytes}}
    if not args.no_staged and headline and w.P == 64:
        # the pages' own four-step form (block states in HBM, a separate state
        # pass) at the same shape, as an explicit choice: not the headline value
        _, sp = time_scan(w, max(10, args.steps // 5), 3, device, algo="staged")
        smean = sum(sp) / len(sp)
        nc = -(-w.L // w.chunk)
        # the state pass reads every block's local state and the initial state,
        # and writes every block's entering state and the final state
        state_bytes = 2 * w.B * (nc + 1) * w.H * w.P * w.N * 4
        extra["staged"] = {"workload": WORKLOAD_NAMES.get(w.name, w.name) + "_staged_form", "chunk": w.chunk,
                           "us_per_call": smean * 1000.0, "us_median": sp[len(sp) // 2] * 1000.0,
                           "tokens_per_s": tokens / (smean * 1e-3),
                           "kernels": f"gram_kernel<{w.N}> + scan_mfma<{w.N}, {w.chunk}, kState> + state_pass_kernel + "
                                      f"scan_mfma<{w.N}, {w.chunk}, kOutput>",
                           "state_pass_bytes": state_bytes,
                           "roofline": {"bound": "hbm", "achieved": byts / (smean * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s", "frac": byts / (smean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes": byts}}
    if not args.no_varlen and headline:
        # timed last before the headline call, whose kernels it shares but for
        # the reset masks, over enough calls (~30 ms) to hold the device at
        # its sustained clocks
        vp, nseq = time_varlen(w, max(200, args.steps // 2), 3, device)
        vmean = sum(vp) / len(vp)
        vb = scan_algorithmic(w)[0] + w.B * w.L * 4      # + seq_idx
        extra["varlen"] = {"workload": WORKLOAD_NAMES.get(w.name, w.name) + "_packed_documents",
                           "documents_per_call": nseq, "median_document_tokens": VARLEN_MEAN_LEN,
                           "us_per_call": vmean * 1000.0, "us_median": vp[len(vp) // 2] * 1000.0,
                           "tokens_per_s": tokens / (vmean * 1e-3),
                           "kernels": "mark_resets + prep_kernel<128, true> + pipe_kernel<128, true>",
                           "roofline": {"bound": "hbm", "achieved": vb / (vmean * 1e-3) / 1e9,
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": vb / (vmean * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes": vb}}
    wall, per = time_scan(w, args.steps, args.warmup, device)
    ms_step = wall * 1000.0 / args.steps
    kern_ms = sum(per) / len(per)
    achieved = byts / (kern_ms * 1e-3) / 1e9
    metric = HEADLINE_METRIC if headline else \
        f"SSD chunk-scan fwd tokens/s at {WORKLOAD_DESC.get(w.name, w.name)}; % of roofline"
    kernels = (f"gram tiles (gram_kernel, or prep_kernel<{w.N}> with the segment states) + pipe_kernel<{w.N}>"
               if per_sequence_scan(w) else "staged or reference kernels")
    out = {
        "metric": metric,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES.get(w.name, w.name), "batch": w.B, "seq_len": w.L,
                   "heads": w.H, "head_dim": w.P, "state": w.N, "groups": w.G, "chunk": w.chunk,
                   "block_tokens": block, "init_state": bool(w.init), "parallelism": "single_gpu"},
        "kernel_ms": {"mean": kern_ms, "median": per[len(per) // 2], "p10": per[len(per) // 10],
                      "p90": per[(9 * len(per)) // 10]},
        "roofline": {"bound": "hbm", "kernels": kernels + " (one ssd_chunk_scan_fwd call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": scan_traffic(args.workload),
                     "algorithmic_bytes": byts, "algorithmic_flops": flops, "flops_block_tokens": block,
                     "mfma_frac": flops / (kern_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
    }
    out["roofline"]["copy_gbs"] = copy_gbs
    out["roofline"]["frac_of_copy"] = achieved / copy_gbs
    out["timed_after"] = ["copy"] + list(extra)
    out.update(extra)
    if not args.no_cpu_baseline and headline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
