"""GPU parity of ssd_chunk_scan_fwd against the fp64 oracle, through the C ABI.

Every case prints its name, shape and algorithm before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, gpu_scan, oracle_scan, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu

MFMA_ALGOS = ["reference", "staged", "pipe"]

# (name, B, L, H, P, N, G, chunk, dtype, init, regime, algos)
SMALL = [
    ("tiny_fp32", 1, 256, 4, 16, 16, 1, 64, "fp32", False, "default", ["reference", "auto"]),
    ("fp32_ragged_groups", 2, 130, 4, 32, 32, 2, 64, "fp32", True, "long_memory", ["reference"]),
    ("fp32_wide", 1, 70, 2, 128, 256, 1, 256, "fp32", True, "default", ["reference"]),
    ("bf16_p16", 1, 200, 2, 16, 16, 1, 64, "bf16", True, "default", ["reference", "auto"]),
    ("bf16_one_token", 2, 1, 4, 64, 128, 1, 256, "bf16", True, "default", MFMA_ALGOS),
    ("bf16_ragged_init", 2, 300, 4, 64, 128, 1, 256, "bf16", True, "default", MFMA_ALGOS),
    ("bf16_long_memory_q64", 1, 1000, 3, 64, 64, 1, 64, "bf16", False, "long_memory", MFMA_ALGOS),
    ("bf16_no_decay_groups_n256", 2, 513, 4, 64, 256, 2, 128, "bf16", True, "no_decay", MFMA_ALGOS),
    ("bf16_n256_long_memory", 2, 1100, 4, 64, 256, 1, 256, "bf16", True, "long_memory", MFMA_ALGOS),
    ("bf16_n256_decay_bursts_q64", 1, 900, 2, 64, 256, 1, 64, "bf16", True, "decay_bursts", MFMA_ALGOS),
    ("bf16_n256_one_token", 2, 1, 2, 64, 256, 1, 256, "bf16", False, "default", MFMA_ALGOS),
    ("bf16_long_memory_n128_q128", 2, 777, 6, 64, 128, 3, 128, "bf16", True, "long_memory", MFMA_ALGOS),
    ("bf16_many_chunks", 1, 4100, 2, 64, 128, 1, 64, "bf16", True, "long_memory", MFMA_ALGOS),
    # stretches of very strong decay next to ordinary ones
    ("bf16_decay_bursts", 2, 1500, 4, 64, 128, 1, 256, "bf16", True, "decay_bursts", MFMA_ALGOS),
    ("bf16_strong_decay_n64_groups", 1, 700, 4, 64, 64, 2, 64, "bf16", True, "strong_decay", MFMA_ALGOS),
    # long runs of ordinary decay
    ("bf16_default_long", 1, 3000, 2, 64, 128, 1, 256, "bf16", True, "default", MFMA_ALGOS),
    # head dim 128 (two heads of 64 channels sharing dt, A and D on the matrix cores)
    ("bf16_p128_ragged", 2, 700, 4, 128, 128, 1, 256, "bf16", True, "long_memory", ["reference", "pipe", "auto"]),
    ("bf16_p128_n256_groups", 1, 600, 4, 128, 256, 2, 128, "bf16", True, "default", ["reference", "pipe"]),
    ("bf16_p128_n64_bursts", 1, 1000, 6, 128, 64, 3, 64, "bf16", False, "decay_bursts", ["reference", "pipe"]),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_match_oracle(case):
    name, B, L, H, P, N, G, Q, dtype, init, regime, algos = case
    d = si.make_scan_inputs(B, L, H, P, N, G, dtype=dtype, init=init, seed=1000 + L, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, dtype)
    for algo in algos:
        announce(f"{name} B{B} L{L} H{H} P{P} N{N} G{G} Q{Q} {dtype} algo={algo}")
        y, fin = gpu_scan(dd, Q, algo=algo)
        ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
        print(f"    y err {ey:.3e}  final err {ef:.3e}", flush=True)
        assert ey <= TOL[dtype], (algo, ey)
        assert ef <= TOL[dtype], (algo, ef)


WORKLOADS = ["tiny_fp32", "m2_130m", "m2_2p7b", "long_n128", "long_n256", "m2_2p7b_p128"]


@pytest.mark.parametrize("wname", WORKLOADS)
def test_workloads_match_oracle(wname):
    """Full-size workloads, in the launch configuration the benchmark times
    (algo auto).  The long sequences check a sample of heads."""
    w = si.WORKLOADS[wname]
    d = si.workload_scan_inputs(w)
    dd = to_device(d, w.dtype)
    announce(f"{wname} B{w.B} L{w.L} H{w.H} P{w.P} N{w.N} Q{w.chunk} {w.dtype} algo=auto")
    y, fin = gpu_scan(dd, w.chunk)
    bh = None
    if w.L > 10000:
        bh = [0, 5, 11, 23]
    y_ref, f_ref = oracle_scan(d, bh=bh)
    y_np, f_np = to_np(y), to_np(fin)
    if bh is not None:
        heads = [i % w.H for i in bh]
        y_np, y_ref = y_np[:, :, heads], y_ref[:, :, heads]
        f_np, f_ref = f_np[:, heads], f_ref[:, heads]
    ey, ef = rel_err(y_np, y_ref), rel_err(f_np, f_ref)
    print(f"    y err {ey:.3e}  final err {ef:.3e}", flush=True)
    assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]


def test_chunk_size_independence_on_gpu():
    B, L, H, P, N = 2, 700, 4, 64, 128
    d = si.make_scan_inputs(B, L, H, P, N, 1, dtype="bf16", init=True, seed=77, regime="long_memory")
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    outs = []
    for Q in (64, 128, 256):
        for algo in ("staged", "pipe"):
            announce(f"chunk independence Q{Q} algo={algo}")
            y, fin = gpu_scan(dd, Q, algo=algo)
            outs.append((to_np(y), to_np(fin)))
            assert rel_err(outs[-1][0], y_ref) <= 2e-2
            assert rel_err(outs[-1][1], f_ref) <= 2e-2
    for y, fin in outs[1:]:
        assert rel_err(y, outs[0][0]) <= 2e-2 and rel_err(fin, outs[0][1]) <= 2e-2


@pytest.mark.parametrize("algo", ["reference", "staged", "pipe"])
def test_split_resume_on_gpu(algo):
    """Running the first k tokens, then the rest from the returned state,
    matches one run over the whole sequence."""
    B, L, H, P, N, k = 2, 900, 4, 64, 128, 333
    d = si.make_scan_inputs(B, L, H, P, N, 1, dtype="bf16", init=True, seed=88, regime="long_memory")
    y_ref, f_ref = oracle_scan(d)
    first = {n: (v[:, :k].copy() if n in ("x", "dt", "Bm", "Cm") else v) for n, v in d.items()}
    rest = {n: (v[:, k:].copy() if n in ("x", "dt", "Bm", "Cm") else v) for n, v in d.items()}
    announce(f"split/resume k={k} algo={algo}")
    y1, f1 = gpu_scan(to_device(first, "bf16"), 128, algo=algo)
    dr = to_device(rest, "bf16")
    dr["init"] = f1
    y2, f2 = gpu_scan(dr, 128, algo=algo)
    y = np.concatenate([to_np(y1), to_np(y2)], axis=1)
    assert rel_err(y, y_ref) <= 2e-2
    assert rel_err(to_np(f2), f_ref) <= 2e-2


def test_pipe_is_deterministic():
    # the segmented launch (80 sequences < 256 compute units) and a plain one
    for (B, L, H) in ((2, 2048, 40), (2, 700, 300)):
        d = si.make_scan_inputs(B, L, H, 64, 128, 1, dtype="bf16", init=True, seed=5)
        dd = to_device(d, "bf16")
        announce(f"pipe determinism B{B} L{L} H{H}")
        y1, f1 = gpu_scan(dd, 256, algo="pipe")
        y2, f2 = gpu_scan(dd, 256, algo="pipe")
        assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_empty_inputs():
    import selective_state_space_chunk_amd as ssd
    announce("empty L=0 and B=0")
    H, P, N = 4, 64, 128
    x = torch.zeros((2, 0, H, P), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((2, 0, H), device="cuda")
    A = -torch.ones(H, device="cuda")
    Bm = torch.zeros((2, 0, 1, N), dtype=torch.bfloat16, device="cuda")
    D = torch.ones(H, device="cuda")
    init = torch.randn((2, H, P, N), device="cuda")
    y, fin = ssd.ssd_chunk_scan_fwd(x, dt, A, Bm, Bm, D, init, 256)
    torch.cuda.synchronize()
    assert y.shape == x.shape and torch.equal(fin, init)
    y, fin = ssd.ssd_chunk_scan_fwd(x, dt, A, Bm, Bm, D, None, 256)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin) == 0
    xb = torch.zeros((0, 5, H, P), dtype=torch.bfloat16, device="cuda")
    y, fin = ssd.ssd_chunk_scan_fwd(xb, torch.zeros((0, 5, H), device="cuda"), A,
                                    torch.zeros((0, 5, 1, N), dtype=torch.bfloat16, device="cuda"),
                                    torch.zeros((0, 5, 1, N), dtype=torch.bfloat16, device="cuda"),
                                    D, None, 256)
    torch.cuda.synchronize()
    assert y.shape == xb.shape and fin.shape == (0, H, P, N)


def test_one_workspace_serves_different_shapes():
    """One workspace, large enough for every call, serves calls of different
    shapes and algorithms one after another: each call's scratch (block
    states, gram tiles, segment states) is written before it is read, so
    nothing a call leaves behind reaches the next."""
    import selective_state_space_chunk_amd as ssd
    calls = [((4, 1500, 8, 256, 64), "staged"), ((3, 700, 10, 128, 128), "pipe"), ((1, 300, 2, 64, 64), "pipe"),
             ((4, 1500, 8, 128, 64), "staged"), ((1, 5000, 3, 128, 256), "pipe"), ((2, 400, 6, 64, 128), "reference")]
    nbytes = max(ssd.ssd_chunk_scan_workspace_size(B, L, H, 64, 1, N, Q, torch.bfloat16, algo)
                 for (B, L, H, N, Q), algo in calls)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bit patterns
    for (B, L, H, N, Q), algo in calls:
        d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=902 + L, regime="long_memory")
        announce(f"shared workspace: {algo} B{B} L{L} H{H} N{N} Q{Q}")
        y, fin = gpu_scan(to_device(d, "bf16"), Q, algo=algo, workspace_tensor=ws)
        y_ref, f_ref = oracle_scan(d)
        assert rel_err(to_np(y), y_ref) <= 2e-2
        assert rel_err(to_np(fin), f_ref) <= 2e-2


def test_workspace_is_sized_for_the_algorithm_run():
    """A workspace of exactly the size the query gives is enough, one byte less
    is refused before anything is launched; the per-sequence scan needs no
    per-block states."""
    import selective_state_space_chunk_amd as ssd
    B, L, H, N = 2, 1000, 6, 128
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=31, regime="long_memory")
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    for algo in ("auto", "pipe", "staged", "reference"):
        nbytes = ssd.ssd_chunk_scan_workspace_size(B, L, H, 64, 1, N, 256, torch.bfloat16, algo)
        announce(f"exact workspace {algo}: {nbytes} bytes")
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        y, fin = gpu_scan(dd, 256, algo=algo, workspace_tensor=ws)
        assert rel_err(to_np(y), y_ref) <= 2e-2 and rel_err(to_np(fin), f_ref) <= 2e-2
        with pytest.raises(ssd.SSDError) as ei:
            gpu_scan(dd, 256, algo=algo, workspace_tensor=ws[:nbytes - 1])
        assert ei.value.status == ssd.SSD_ERR_WORKSPACE


def test_calls_on_two_streams_use_their_own_workspaces():
    """The binding's cached workspace is per (device, stream): two scans in
    flight at once on two streams do not share scratch."""
    import selective_state_space_chunk_amd as ssd
    shapes = [(2, 3000, 40, 128), (1, 2500, 30, 64)]   # both cut into time segments
    data, refs = [], []
    for i, (B, L, H, N) in enumerate(shapes):
        d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=61 + i, regime="long_memory")
        data.append(to_device(d, "bf16"))
        refs.append(oracle_scan(d))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for i, (dd, s) in enumerate(zip(data, streams)):
            announce(f"stream {i} call {rep}")
            with torch.cuda.stream(s):
                outs.append((i, ssd.ssd_chunk_scan_fwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"],
                                                       dd["init"], 256, stream=s)))
    torch.cuda.synchronize()
    for i, (y, fin) in outs:
        assert rel_err(to_np(y), refs[i][0]) <= 2e-2 and rel_err(to_np(fin), refs[i][1]) <= 2e-2


@pytest.mark.parametrize("N,Q", [(128, 64), (128, 128), (128, 256), (64, 64), (256, 128)])
def test_nothing_is_read_past_the_sequence_end(N, Q):
    """x, dt, Bm and Cm are the first L rows of buffers whose remaining rows
    hold NaN; a read past token L-1 (the ragged tail of the last block) would
    make outputs non-finite."""
    import selective_state_space_chunk_amd as ssd
    B, L, H, P, extra = 1, 3 * Q + 5, 4, 64, 300
    d = si.make_scan_inputs(B, L, H, P, N, 1, dtype="bf16", init=True, seed=4242 + Q + N, regime="long_memory")
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")

    def padded(t):
        big = torch.full((B, L + extra) + tuple(t.shape[2:]), float("nan"), dtype=t.dtype, device=t.device)
        big[:, :L] = t
        return big[:, :L]

    for name in ("x", "dt", "Bm", "Cm"):
        dd[name] = padded(dd[name])
        assert dd[name].is_contiguous()
    algos = ["reference", "staged", "pipe"]
    for algo in algos:
        announce(f"NaN past the end N{N} Q{Q} L{L} algo={algo}")
        y = torch.full_like(dd["x"], float("nan"))
        fin = torch.full((B, H, P, N), float("nan"), device="cuda")
        ssd.ssd_chunk_scan_fwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], dd["init"], Q,
                               y=y, final_state=fin, algo=algo)
        torch.cuda.synchronize()
        assert rel_err(to_np(y), y_ref) <= 2e-2
        assert rel_err(to_np(fin), f_ref) <= 2e-2


# More (batch, head) sequences than compute units (256 on MI355X) but fewer
# than twice as many: the pipe algorithm runs one sequence whole per
# workgroup and spreads the rest as segments over all workgroups, with the
# segments' entering states from a first kernel.  (B, H, L, N, regime, init)
BALANCED = [
    (1, 300, 1024, 128, "long_memory", True),
    (2, 150, 320, 64, "default", True),
    (1, 257, 64 * 9 + 5, 128, "default", False),
    (1, 300, 65, 128, "long_memory", True),
    (1, 300, 700, 256, "long_memory", True),
    (2, 140, 64 * 5 + 3, 256, "default", False),
]


@pytest.mark.parametrize("case", BALANCED, ids=[f"B{c[0]}_H{c[1]}_L{c[2]}_N{c[3]}" for c in BALANCED])
def test_more_sequences_than_compute_units(case):
    B, H, L, N, regime, init = case
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=init, seed=900 + H, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    announce(f"balanced B{B} H{H} L{L} N{N} {regime} algo=pipe")
    for rep in range(2):
        y, fin = gpu_scan(dd, 256, algo="pipe")
        ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
        print(f"    call {rep}: y err {ey:.3e}  final err {ef:.3e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


# At most half as many (batch, head) sequences as compute units: the pipe
# algorithm cuts every sequence into time segments, one workgroup each, the
# entering state of each from the segment states of a first kernel.
# (B, H, L, N, regime, init)
FEW_LONG = [
    (1, 1, 64 * 300 + 7, 128, "long_memory", True),
    (1, 2, 3000, 64, "default", False),
    (2, 3, 5000, 128, "long_memory", True),
    # 767 sub-blocks over 256 workgroups: segments of 3 sub-blocks (a pair and
    # a lone one), the last ragged
    (1, 1, 767 * 64 - 5, 64, "default", True),
    (1, 3, 5000, 256, "long_memory", True),
    (1, 1, 64 * 40 + 9, 256, "default", True),
    (2, 5, 3000, 256, "decay_bursts", True),
]


@pytest.mark.parametrize("case", FEW_LONG, ids=[f"B{c[0]}_H{c[1]}_L{c[2]}_N{c[3]}" for c in FEW_LONG])
def test_few_long_sequences_are_cut_into_segments(case):
    B, H, L, N, regime, init = case
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=init, seed=1700 + H + L, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    announce(f"segmented B{B} H{H} L{L} N{N} {regime} algo=pipe")
    for rep in range(2):
        y, fin = gpu_scan(dd, 256, algo="pipe")
        ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
        print(f"    call {rep}: y err {ey:.3e}  final err {ef:.3e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


# The other two launch regimes of the pipe algorithm on a device of C compute
# units (256 on MI355X): at least 2C (batch, head) sequences, one workgroup
# each in several rounds; between C/2 and C sequences, one workgroup each
# with some compute units idle.  (B, H, L, N, regime, init)
ONE_PER_SEQUENCE = [
    (2, 300, 200, 64, "default", True),
    (4, 160, 64 * 2 + 3, 128, "decay_bursts", False),
    (1, 200, 300, 128, "long_memory", True),
    (2, 97, 64 * 3 + 1, 256, "default", True),
]


@pytest.mark.parametrize("case", ONE_PER_SEQUENCE, ids=[f"B{c[0]}_H{c[1]}_L{c[2]}_N{c[3]}" for c in ONE_PER_SEQUENCE])
def test_one_workgroup_per_sequence_regimes(case):
    B, H, L, N, regime, init = case
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=init, seed=2300 + H + L, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    announce(f"one per sequence B{B} H{H} L{L} N{N} {regime} algo=pipe")
    y, fin = gpu_scan(dd, 256, algo="pipe")
    ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
    print(f"    y err {ey:.3e}  final err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


# Head dim 128 in the launch shapes of the per-sequence scan: few sequences
# cut into segments, more sequences than compute units, one token.
# (B, L, H, N, regime, init); P = 128
P128 = [
    (1, 3000, 2, 128, "long_memory", True),
    (1, 700, 150, 64, "default", True),
    (2, 5000, 3, 256, "long_memory", False),
    (3, 1, 4, 128, "default", True),
]


@pytest.mark.parametrize("case", P128, ids=[f"B{c[0]}_L{c[1]}_H{c[2]}_N{c[3]}" for c in P128])
def test_head_dim_128_launch_shapes(case):
    B, L, H, N, regime, init = case
    d = si.make_scan_inputs(B, L, H, 128, N, 1, dtype="bf16", init=init, seed=1900 + H + L, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    announce(f"P128 B{B} L{L} H{H} N{N} {regime} algo=pipe")
    y, fin = gpu_scan(dd, 256, algo="pipe")
    ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
    print(f"    y err {ey:.3e}  final err {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]
