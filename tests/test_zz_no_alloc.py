"""ssd_chunk_scan_fwd_noalloc (the scan with the library's static per-device
scratch, for callers that cannot allocate) against ssd_chunk_scan_fwd, through
the C ABI.

The two entry points run the same kernels on the same inputs, so their outputs
must be identical; both are also held to the fp64 oracle.  Calls come in a row
on one device, each smaller than the one before, so that each finds the last
call's scratch in the array.  Every case prints its name and shape first.
"""
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, oracle_scan, rel_err, to_device, to_np

pytestmark = pytest.mark.gpu

# (B, L, H, N, G, chunk, regime), each input smaller than the one before: a
# plain launch with one workgroup per sequence (gram tiles in the scratch),
# then two calls whose sequences are cut into time segments (segment states
# in the scratch as well)
CALLS = [
    (1, 2000, 200, 64, 2, 128, "default"),
    (2, 3000, 40, 128, 1, 256, "long_memory"),
    (1, 700, 6, 64, 1, 64, "long_memory"),
]


def test_no_alloc_matches_the_allocating_entry_point():
    import selective_state_space_chunk_amd as ssd
    for B, L, H, N, G, Q, regime in CALLS:
        d = si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=True, seed=7100 + L, regime=regime)
        dd = to_device(d, "bf16")
        need = ssd.ssd_chunk_scan_workspace_size(B, L, H, 64, G, N, Q, torch.bfloat16)
        assert 0 < need <= ssd.NOALLOC_SCRATCH_BYTES
        announce(f"no-alloc B{B} L{L} H{H} N{N} G{G} Q{Q} {regime} (workspace {need} bytes)")
        y_ref, f_ref = ssd.ssd_chunk_scan_fwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"],
                                              dd["init"], Q)
        y = torch.full_like(dd["x"], float("nan"))
        fin = torch.full((B, H, 64, N), float("nan"), device="cuda")
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        ssd.ssd_chunk_scan_fwd_noalloc(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], dd["init"], Q,
                                       y, fin)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(y, y_ref) and torch.equal(fin, f_ref)
        yo, fo = oracle_scan(d)
        assert rel_err(to_np(y), yo) <= TOL["bf16"] and rel_err(to_np(fin), fo) <= TOL["bf16"]


def test_no_alloc_refuses_shapes_beyond_its_scratch():
    import selective_state_space_chunk_amd as ssd
    # float32 runs the reference kernels, whose block states need 33.6 MB here
    B, L, H, N = 1, 16384, 8, 256
    need = ssd.ssd_chunk_scan_workspace_size(B, L, H, 64, 1, N, 256, torch.float32)
    assert need > ssd.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, L, H, 64), dtype=torch.float32, device="cuda")
    bm = torch.zeros((B, L, 1, N), dtype=torch.float32, device="cuda")
    announce(f"no-alloc refuses fp32 B{B} L{L} H{H} N{N} (workspace {need} bytes)")
    with pytest.raises(ssd.SSDError) as ei:
        ssd.ssd_chunk_scan_fwd_noalloc(x, torch.zeros((B, L, H), device="cuda"), -torch.ones(H, device="cuda"),
                                       bm, bm, torch.zeros(H, device="cuda"), None, 256, torch.empty_like(x))
    assert ei.value.status == ssd.SSD_ERR_TOO_LARGE
    # and, after the refusal, a call that fits still runs
    d = si.make_scan_inputs(1, 300, 4, 64, 128, 1, dtype="bf16", init=False, seed=7200)
    dd = to_device(d, "bf16")
    y = torch.empty_like(dd["x"])
    ssd.ssd_chunk_scan_fwd_noalloc(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], None, 256, y)
    torch.cuda.synchronize()
    yo, _ = oracle_scan(d)
    assert rel_err(to_np(y), yo) <= TOL["bf16"]
