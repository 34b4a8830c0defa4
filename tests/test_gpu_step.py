"""GPU parity of ssd_step against the fp64 oracle, through the C ABI, and the
decode path cross-checked against the chunk scan on the same sequence."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
from gpu_util import TOL, announce, rel_err, to_np

pytestmark = pytest.mark.gpu


def dev_step_inputs(s, dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to("cuda", dtype=td if k in ("x", "Bm", "Cm") else torch.float32)
            for k, v in s.items()}


@pytest.mark.parametrize("shape", [(3, 4, 16, 1, 16), (2, 6, 32, 3, 64), (4, 2, 128, 1, 256),
                                   (5, 8, 64, 2, 128)])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_step_small_shapes(shape, dtype):
    import selective_state_space_chunk_amd as ssd
    B, H, P, G, N = shape
    st_np = si.make_step_state(B, H, P, N, seed=3).astype(np.float64)
    st = torch.from_numpy(st_np).float().cuda()
    ref_state = st_np.copy()
    for t in range(5):
        s = si.make_step_inputs(B, H, P, N, G, step=t, dtype=dtype, seed=3)
        announce(f"step B{B} H{H} P{P} G{G} N{N} {dtype} t={t}")
        dd = dev_step_inputs(s, dtype)
        y = ssd.ssd_step(st, dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"])
        torch.cuda.synchronize()
        f = si.as_f64(s)
        y_ref = oracle.step(ref_state, f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"])
        assert rel_err(to_np(y), y_ref) <= TOL[dtype]
    assert rel_err(to_np(st), ref_state) <= TOL[dtype]


@pytest.mark.timeout(900)
def test_decode_workload_1024_steps():
    """The decode workload: B=256, H=80, P=64, N=128, 1024 consecutive tokens
    from a random state; oracle on a sample of (b, h) pairs; then the same
    1024-token sequence through the chunk scan (first 8 batch rows) must give
    the same outputs and final state."""
    import selective_state_space_chunk_amd as ssd
    w = si.WORKLOADS["decode_2p7b"]
    B, H, P, N, G, T = w.B, w.H, w.P, w.N, w.G, w.steps
    st0 = si.make_step_state(B, H, P, N, seed=w.seed)
    st = torch.from_numpy(st0).cuda()
    sample = [0, 81, 1000, 5555, 12345, 20479]
    ref_state = np.zeros((B, H, P, N))
    ref_state.reshape(B * H, P, N)[sample] = st0.reshape(B * H, P, N)[sample]
    Bs = 8                                      # batch rows re-run through the chunk scan
    xs = np.zeros((Bs, T, H, P), np.float32)
    dts = np.zeros((Bs, T, H), np.float32)
    bms = np.zeros((Bs, T, G, N), np.float32)
    cms = np.zeros((Bs, T, G, N), np.float32)
    ys = np.zeros((Bs, T, H, P))
    worst = 0.0
    announce(f"decode B{B} H{H} P{P} N{N} x {T} steps")
    for t in range(T):
        s = si.make_step_inputs(B, H, P, N, G, step=t, dtype="bf16", seed=w.seed)
        dd = dev_step_inputs(s, "bf16")
        y = ssd.ssd_step(st, dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"])
        f = si.as_f64(s)
        y_ref = oracle.step(ref_state, f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], bh=sample)
        y_np = to_np(y)
        yr = y_ref.reshape(B * H, P)[sample]
        worst = max(worst, rel_err(y_np.reshape(B * H, P)[sample], yr))
        xs[:, t], dts[:, t], bms[:, t], cms[:, t] = s["x"][:Bs], s["dt"][:Bs], s["Bm"][:Bs], s["Cm"][:Bs]
        ys[:, t] = y_np[:Bs]
        if t % 256 == 0:
            print(f"    step {t}: worst y err so far {worst:.3e}", flush=True)
    torch.cuda.synchronize()
    assert worst <= 2e-2, worst
    st_np = to_np(st)
    assert rel_err(st_np.reshape(B * H, P, N)[sample], ref_state.reshape(B * H, P, N)[sample]) <= 2e-2

    # the same sequence through the chunk scan
    announce("decode cross-check through the chunk scan, 8 batch rows")
    td = torch.bfloat16
    yc, fc = ssd.ssd_chunk_scan_fwd(torch.from_numpy(xs).to("cuda", td), torch.from_numpy(dts).cuda(),
                                    dd["A"], torch.from_numpy(bms).to("cuda", td),
                                    torch.from_numpy(cms).to("cuda", td), dd["D"],
                                    torch.from_numpy(st0[:Bs]).cuda(), w.chunk)
    torch.cuda.synchronize()
    assert rel_err(to_np(yc), ys) <= 2e-2
    assert rel_err(to_np(fc), st_np[:Bs]) <= 2e-2
