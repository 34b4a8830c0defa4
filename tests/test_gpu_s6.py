"""GPU parity of ssd_selective_scan (Mamba-1 selective scan, diagonal A)
against the fp64 oracle (oracle/s6.py), through the C ABI.

y (bfloat16) and the final state (fp32) are compared with gpu_util.rel_err at
2e-2.  At the Mamba-1 2.8B layer shape the oracle runs on sampled channels.
Every case prints its name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, rel_err, to_np

from oracle.s6 import selective_scan

pytestmark = pytest.mark.gpu


def _dev(d):
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
        elif k in ("x", "dt", "Bm", "Cm"):
            out[k] = torch.from_numpy(v).to("cuda", dtype=torch.bfloat16)
        else:
            out[k] = torch.from_numpy(v).to("cuda")
    return out


def _gpu(dd, zoh):
    import selective_state_space_chunk_amd as ssd
    y, fin = ssd.ssd_selective_scan(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], dd["init"], zoh=zoh)
    torch.cuda.synchronize()
    return to_np(y), to_np(fin)


# (name, B, L, Dch, N, G, zoh, init)
CASES = [
    ("zoh_n16", 2, 100, 128, 16, 1, True, True),
    ("simple_term_groups", 1, 70, 256, 16, 2, False, True),
    ("n8_ragged_no_init", 2, 33, 64, 8, 1, True, False),
    ("n32", 1, 65, 128, 32, 1, True, True),
    ("one_token", 1, 1, 64, 16, 1, True, True),
    ("several_chunks", 1, 300, 192, 16, 3, True, True),
    ("n8_simple_term", 1, 40, 64, 8, 1, False, True),
    ("n32_simple_term", 1, 50, 64, 32, 1, False, False),
]


@pytest.mark.parametrize("N", [16, 32])
def test_zero_decay_states_take_the_limit(N):
    # A = 0 for some states: the zero-order-hold term is its limit dt Bm x there
    B, L, Dch = 1, 90, 64
    d = si.make_s6_inputs(B, L, Dch, N, 1, init=True, seed=6401 + N)
    d["A"][::3, ::2] = 0.0
    f = si.as_f64(d)
    y_ref, f_ref = selective_scan(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], zoh=True)
    announce(f"selective scan with zero decays: B{B} L{L} Dch{Dch} N{N}")
    y, fin = _gpu(_dev(d), True)
    ey, ef = rel_err(y, y_ref), rel_err(fin, f_ref)
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_selective_scan_matches_oracle(case):
    name, B, L, Dch, N, G, zoh, init = case
    d = si.make_s6_inputs(B, L, Dch, N, G, init=init, seed=6100 + L + Dch)
    f = si.as_f64(d)
    y_ref, f_ref = selective_scan(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], zoh=zoh)
    announce(f"selective scan {name}: B{B} L{L} Dch{Dch} N{N} G{G} zoh={zoh} init={init}")
    y, fin = _gpu(_dev(d), zoh)
    ey, ef = rel_err(y, y_ref), rel_err(fin, f_ref)
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_full_size_sampled_channels():
    B, L, Dch, N = 4, 4096, 5120, 16
    d = si.make_s6_inputs(B, L, Dch, N, 1, init=True, seed=6201)
    ch = [0, 1, 63, 64, 2555, 5119]
    f = si.as_f64(d)
    y_ref, f_ref = selective_scan(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], zoh=True, channels=ch)
    announce(f"selective scan full size: B{B} L{L} Dch{Dch} N{N}, channels {ch}")
    y, fin = _gpu(_dev(d), True)
    ey, ef = rel_err(y[:, :, ch], y_ref[:, :, ch]), rel_err(fin[:, ch], f_ref[:, ch])
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_without_tokens_and_uncovered_shapes():
    import selective_state_space_chunk_amd as ssd
    announce("selective scan: L = 0; N = 12 and Dch = 96 are not covered")
    init = torch.randn(2, 64, 16, device="cuda")
    e = torch.empty((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    bm = torch.empty((2, 0, 1, 16), dtype=torch.bfloat16, device="cuda")
    _, fin = ssd.ssd_selective_scan(e, e, -torch.ones(64, 16, device="cuda"), bm, bm, None, init)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)
    for Dch, N in ((64, 12), (96, 16)):
        d = _dev(si.make_s6_inputs(1, 8, Dch, N, 1, seed=6301))
        with pytest.raises(ssd.SSDError) as ei:
            _gpu(d, True)
        assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED


def test_mamba1_130m_shape_sampled_channels():
    # Mamba-1 130M layer: d_inner 1536 channels, N 16; batch 8 of 2048 tokens
    B, L, Dch, N = 8, 2048, 1536, 16
    d = si.make_s6_inputs(B, L, Dch, N, 1, init=True, seed=6501)
    ch = [0, 15, 16, 767, 1535]
    f = si.as_f64(d)
    y_ref, f_ref = selective_scan(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], zoh=True, channels=ch)
    announce(f"selective scan at the Mamba-1 130M shape: B{B} L{L} Dch{Dch} N{N}, channels {ch}")
    y, fin = _gpu(_dev(d), True)
    ey, ef = rel_err(y[:, :, ch], y_ref[:, :, ch]), rel_err(fin[:, ch], f_ref[:, ch])
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)
