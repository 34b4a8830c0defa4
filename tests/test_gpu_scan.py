"""GPU parity of ssd_chunk_scan_fwd against the fp64 oracle, through the C ABI.

Every case prints its name, shape and algorithm before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, gpu_scan, oracle_scan, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu

MFMA_ALGOS = ["reference", "staged", "fused", "chain", "pipe", "pair"]


def covers(algo, H, G):
    """The pair algorithm takes heads two at a time within one group."""
    return algo != "pair" or (H % 2 == 0 and (H // G) % 2 == 0)

# (name, B, L, H, P, N, G, chunk, dtype, init, regime, algos)
SMALL = [
    ("tiny_fp32", 1, 256, 4, 16, 16, 1, 64, "fp32", False, "default", ["reference", "auto"]),
    ("fp32_ragged_groups", 2, 130, 4, 32, 32, 2, 64, "fp32", True, "long_memory", ["reference"]),
    ("fp32_wide", 1, 70, 2, 128, 256, 1, 256, "fp32", True, "default", ["reference"]),
    ("bf16_p16", 1, 200, 2, 16, 16, 1, 64, "bf16", True, "default", ["reference", "auto"]),
    ("bf16_one_token", 2, 1, 4, 64, 128, 1, 256, "bf16", True, "default", MFMA_ALGOS),
    ("bf16_ragged_init", 2, 300, 4, 64, 128, 1, 256, "bf16", True, "default", MFMA_ALGOS),
    ("bf16_long_memory_q64", 1, 1000, 3, 64, 64, 1, 64, "bf16", False, "long_memory", MFMA_ALGOS),
    ("bf16_no_decay_groups_n256", 2, 513, 4, 64, 256, 2, 128, "bf16", True, "no_decay", ["reference", "staged", "auto"]),
    ("bf16_long_memory_n128_q128", 2, 777, 6, 64, 128, 3, 128, "bf16", True, "long_memory", MFMA_ALGOS),
    ("bf16_many_chunks", 1, 4100, 2, 64, 128, 1, 64, "bf16", True, "long_memory", MFMA_ALGOS),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes_match_oracle(case):
    name, B, L, H, P, N, G, Q, dtype, init, regime, algos = case
    d = si.make_scan_inputs(B, L, H, P, N, G, dtype=dtype, init=init, seed=1000 + L, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, dtype)
    for algo in [a for a in algos if covers(a, H, G)]:
        announce(f"{name} B{B} L{L} H{H} P{P} N{N} G{G} Q{Q} {dtype} algo={algo}")
        y, fin = gpu_scan(dd, Q, algo=algo)
        ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
        print(f"    y err {ey:.3e}  final err {ef:.3e}", flush=True)
        assert ey <= TOL[dtype], (algo, ey)
        assert ef <= TOL[dtype], (algo, ef)


WORKLOADS = ["tiny_fp32", "m2_130m", "m2_2p7b", "long_n128", "long_n256"]


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
        for algo in ("staged", "fused", "chain", "pipe", "pair"):
            announce(f"chunk independence Q{Q} algo={algo}")
            y, fin = gpu_scan(dd, Q, algo=algo)
            outs.append((to_np(y), to_np(fin)))
            assert rel_err(outs[-1][0], y_ref) <= 2e-2
            assert rel_err(outs[-1][1], f_ref) <= 2e-2
    for y, fin in outs[1:]:
        assert rel_err(y, outs[0][0]) <= 2e-2 and rel_err(fin, outs[0][1]) <= 2e-2


@pytest.mark.parametrize("algo", ["reference", "staged", "fused", "chain", "pipe", "pair"])
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


def test_fused_is_deterministic_and_hands_off_cleanly():
    import selective_state_space_chunk_amd as ssd
    w = si.WORKLOADS["m2_2p7b"]
    d = si.make_scan_inputs(2, 2048, 16, 64, 128, 1, dtype="bf16", init=True, seed=5)
    dd = to_device(d, "bf16")
    announce("fused determinism B2 L2048 H16")
    ws = torch.zeros(ssd.ssd_chunk_scan_workspace_size(2, 2048, 16, 64, 1, 128, 256, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    y1, f1 = gpu_scan(dd, 256, algo="fused", workspace_tensor=ws)
    y2, f2 = gpu_scan(dd, 256, algo="fused", workspace_tensor=ws)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    ssd.ssd_chunk_scan_workspace_check(ws, 2, 2048, 16, 64, 1, 128, 256)
    del w


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
    """Scratch written by one call (states of a large staged scan) must never
    land where a later one-pass call keeps its hand-off counters and flags."""
    import selective_state_space_chunk_amd as ssd
    nbytes = max(ssd.ssd_chunk_scan_workspace_size(4, 1500, 8, 64, 1, 256, 64, torch.bfloat16),
                 ssd.ssd_chunk_scan_workspace_size(3, 700, 10, 64, 1, 128, 128, torch.bfloat16))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    big = si.make_scan_inputs(4, 1500, 8, 64, 256, 1, dtype="bf16", init=True, seed=901)
    announce("shared workspace: staged B4 L1500 H8 N256 Q64")
    gpu_scan(to_device(big, "bf16"), 64, algo="staged", workspace_tensor=ws)
    for shape in [(3, 700, 10, 128, 128), (1, 300, 2, 64, 64), (4, 1500, 8, 128, 64)]:
        B, L, H, N, Q = shape
        d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=902 + L,
                                regime="long_memory")
        announce(f"shared workspace: fused B{B} L{L} H{H} N{N} Q{Q}")
        y, fin = gpu_scan(to_device(d, "bf16"), Q, algo="fused", workspace_tensor=ws)
        ssd.ssd_chunk_scan_workspace_check(ws, B, L, H, 64, 1, N, Q)
        y_ref, f_ref = oracle_scan(d)
        assert rel_err(to_np(y), y_ref) <= 2e-2
        assert rel_err(to_np(fin), f_ref) <= 2e-2


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
    algos = ["reference", "staged"] + (["fused", "chain", "pipe", "pair"] if N <= 128 else [])
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


# Pairs of adjacent heads per workgroup: odd numbers of pairs, several batch
# rows and groups, ragged and sub-block-short sequences, zero initial state.
# (B, L, H, G, N, regime, init)
PAIRS = [
    (1, 64, 2, 1, 128, "default", True),
    (3, 37, 6, 3, 128, "long_memory", True),
    (2, 1000, 10, 1, 64, "long_memory", False),
    (2, 4096 + 17, 4, 2, 128, "long_memory", True),
    (1, 333, 18, 1, 128, "no_decay", True),
]


@pytest.mark.parametrize("case", PAIRS, ids=[f"B{c[0]}_L{c[1]}_H{c[2]}_G{c[3]}_N{c[4]}" for c in PAIRS])
def test_pair_matches_oracle(case):
    B, L, H, G, N, regime, init = case
    d = si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=init, seed=1300 + L + H, regime=regime)
    y_ref, f_ref = oracle_scan(d)
    dd = to_device(d, "bf16")
    announce(f"pair B{B} L{L} H{H} G{G} N{N} {regime} algo=pair")
    for rep in range(2):
        y, fin = gpu_scan(dd, 256, algo="pair")
        ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
        print(f"    call {rep}: y err {ey:.3e}  final err {ef:.3e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


def test_pair_rejects_odd_head_counts():
    import selective_state_space_chunk_amd as ssd
    for H, G in ((3, 1), (6, 6)):
        d = si.make_scan_inputs(1, 100, H, 64, 128, G, dtype="bf16", init=False, seed=7)
        dd = to_device(d, "bf16")
        announce(f"pair unsupported H{H} G{G}")
        with pytest.raises(ssd.SSDError) as ei:
            gpu_scan(dd, 256, algo="pair")
        assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED


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
