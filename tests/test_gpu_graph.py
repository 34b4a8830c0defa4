"""The forward scan captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed, through the C ABI: callers that capture their launches are the ones
the allocation-free entry point is for, and the workspace entry point is
captured the same way with a caller-held workspace.

The library's per-device set-up (its launch attributes, the scratch address)
happens on a first call outside the capture.  Each replay then runs on new
input values copied into the captured buffers, with eager work and a
synchronisation between replays, and must equal an eager call on the same
values bit for bit (the kernels are deterministic); the first replay's values
are also held to the fp64 oracle.  Every case prints its name and shape first.
"""
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, oracle_scan, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu

INPUTS = ("x", "dt", "A", "Bm", "Cm", "D", "init")

# (name, B, L, H, N, G, chunk): one workgroup per sequence (gram tiles, then
# the scan), and more sequences than compute units (segment states and gram
# tiles in one launch, then the scan)
CASES = [
    ("one_workgroup_per_sequence", 1, 700, 6, 128, 1, 256),
    ("segmented", 1, 1100, 300, 64, 1, 256),
]


@pytest.mark.parametrize("entry", ["noalloc", "workspace"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager_calls(case, entry):
    import selective_state_space_chunk_amd as ssd
    name, B, L, H, N, G, Q = case
    buf = to_device(si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=True, seed=7300 + L), "bf16")
    y = torch.empty_like(buf["x"])
    fin = torch.empty((B, H, 64, N), device="cuda")
    ws = None
    if entry == "workspace":
        ws = torch.empty(ssd.ssd_chunk_scan_workspace_size(B, L, H, 64, G, N, Q, torch.bfloat16),
                         dtype=torch.uint8, device="cuda")

    def call():
        if entry == "noalloc":
            ssd.ssd_chunk_scan_fwd_noalloc(buf["x"], buf["dt"], buf["A"], buf["Bm"], buf["Cm"], buf["D"],
                                           buf["init"], Q, y, fin)
        else:
            ssd.ssd_chunk_scan_fwd(buf["x"], buf["dt"], buf["A"], buf["Bm"], buf["Cm"], buf["D"], buf["init"], Q,
                                   y=y, final_state=fin, workspace_tensor=ws)

    announce(f"graph {entry} {name}: B{B} L{L} H{H} N{N} G{G} Q{Q}")
    call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        d = si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=True, seed=7400 + 10 * r + L)
        new = to_device(d, "bf16")
        for k in INPUTS:
            buf[k].copy_(new[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_e, f_e = ssd.ssd_chunk_scan_fwd(new["x"], new["dt"], new["A"], new["Bm"], new["Cm"], new["D"],
                                          new["init"], Q)
        torch.cuda.synchronize()
        print(f"    replay {r}", flush=True)
        assert torch.equal(y, y_e) and torch.equal(fin, f_e), r
        if r == 0:
            yo, fo = oracle_scan(d)
            assert rel_err(to_np(y), yo) <= TOL["bf16"] and rel_err(to_np(fin), fo) <= TOL["bf16"]
