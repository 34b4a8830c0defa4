"""The four-token example of the "Mamba-2" note (section "following four tokens
through once") run through the GPU library, through the C ABI.

The example is a state of size 2 and one channel: h_t = a_t h_{t-1} + B_t x_t,
y_t = C_t . h_t, with the a, B, C and x printed on the page and the outputs
y = [1, 0.5, 4.6, 5.6] printed there (tests/golden/four_token_walkthrough.json).
It is recast in the library's convention the same way as the oracle's pin P1:
A = -1 and dt_t = -ln a_t so that exp(dt_t A) = a_t, and Bm_t = B_t / dt_t so
that dt_t Bm_t = B_t.  The one channel and the two states are zero-padded to
the smallest head dim and state size the library takes; padded channels and
states carry zeros, so channel 0 of y must be the printed outputs.

With an initial state h_{-1} = [1, 1] (decayed by a_0 before token 0), the
outputs worked by hand from the same example are [2.8, 0.95, 4.96, 6.104] and
the final state [6.632, -0.528]; without one the final state is
[6.38, -0.78].

The expected values come from the page (and the hand derivation), not from the
oracle.  float32 mode is held to 1e-4 relative to max |y|; the bfloat16
matrix-core path (x, Bm, Cm rounded to bfloat16) to 2e-2.
"""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import TOL, announce

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "four_token_walkthrough.json")


def padded_inputs(P, N, dtype, init):
    fx = json.load(open(GOLDEN))
    a = np.array(fx["a"], dtype=np.float64)
    dt = (-np.log(a)).astype(np.float32)
    x = np.zeros((1, 4, 1, P), np.float32)
    x[0, :, 0, 0] = fx["x"]
    Bm = np.zeros((1, 4, 1, N), np.float32)
    Bm[0, :, 0, :2] = np.array(fx["B"], np.float64) / dt.astype(np.float64)[:, None]
    Cm = np.zeros((1, 4, 1, N), np.float32)
    Cm[0, :, 0, :2] = fx["C"]
    st = None
    if init is not None:
        st = np.zeros((1, 1, P, N), np.float32)
        st[0, 0, 0, :2] = init
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = "cuda"
    return fx, dict(
        x=torch.from_numpy(x).to(dev, dtype=td), dt=torch.from_numpy(dt.reshape(1, 4, 1)).to(dev),
        A=torch.tensor([-1.0], device=dev), Bm=torch.from_numpy(Bm).to(dev, dtype=td),
        Cm=torch.from_numpy(Cm).to(dev, dtype=td), D=torch.zeros(1, device=dev),
        init=None if st is None else torch.from_numpy(st).to(dev))


# (name, P, N, dtype, algo)
CASES = [
    ("fp32_p16_n16", 16, 16, "fp32", "auto"),
    ("fp32_p16_n16_reference", 16, 16, "fp32", "reference"),
    ("bf16_p64_n128_matrix_cores", 64, 128, "bf16", "auto"),
    ("bf16_p64_n64_matrix_cores", 64, 64, "bf16", "auto"),
]
INITS = [
    (None, [1.0, 0.5, 4.6, 5.6], [6.38, -0.78]),
    ([1.0, 1.0], [2.8, 0.95, 4.96, 6.104], [6.632, -0.528]),
]


@pytest.mark.parametrize("init,y_expect,fin_expect", INITS, ids=["zero_init", "init_1_1"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_four_token_walkthrough_on_gpu(case, init, y_expect, fin_expect):
    import selective_state_space_chunk_amd as ssd
    name, P, N, dtype, algo = case
    fx, d = padded_inputs(P, N, dtype, init)
    if init is None:
        assert y_expect == fx["y_printed_recurrence"]
    announce(f"four-token walkthrough {name}: B1 L4 H1 P{P} N{N} init={init}")
    y, fin = ssd.ssd_chunk_scan_fwd(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], 64, algo=algo)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    fin = fin.cpu().numpy().astype(np.float64)
    tol = TOL[dtype]
    ye = np.array(y_expect)
    err = np.max(np.abs(y[0, :, 0, 0] - ye)) / np.max(np.abs(ye))
    print(f"    y channel 0: {y[0, :, 0, 0]} (err {err:.2e})", flush=True)
    assert err <= tol, err
    # padded channels get nothing: x and the initial state are zero there
    assert np.max(np.abs(y[0, :, 0, 1:])) <= tol * np.max(np.abs(ye))
    fe = np.array(fin_expect)
    ferr = np.max(np.abs(fin[0, 0, 0, :2] - fe)) / np.max(np.abs(fe))
    assert ferr <= tol, ferr
    rest = fin.copy()
    rest[0, 0, 0, :2] = 0.0
    assert np.max(np.abs(rest)) <= tol * np.max(np.abs(fe))


def test_four_token_walkthrough_one_step_at_a_time():
    # the recurrent path (ssd_step): the same example fed one token per call
    import selective_state_space_chunk_amd as ssd
    fx, d = padded_inputs(16, 16, "fp32", None)
    state = torch.zeros((1, 1, 16, 16), device="cuda")
    announce("four-token walkthrough through ssd_step, fp32, P16 N16")
    ys = []
    for t in range(4):
        # fresh (16-byte aligned) tensors for the one token's inputs
        y = ssd.ssd_step(state, d["x"][:, t].clone(), d["dt"][:, t].clone(), d["A"],
                         d["Bm"][:, t].clone(), d["Cm"][:, t].clone(), d["D"])
        torch.cuda.synchronize()
        ys.append(float(y[0, 0, 0]))
    ye = np.array(fx["y_printed_recurrence"])
    err = np.max(np.abs(np.array(ys) - ye)) / np.max(np.abs(ye))
    print(f"    y: {ys} (err {err:.2e})", flush=True)
    assert err <= TOL["fp32"], err
    fin = state.cpu().numpy().astype(np.float64)[0, 0, 0, :2]
    assert np.max(np.abs(fin - np.array([6.38, -0.78]))) / 6.38 <= TOL["fp32"]
