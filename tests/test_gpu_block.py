"""GPU parity of the block prologue (ssd_block_prologue) and the gated norm
(ssd_gated_norm) against the fp64 oracle (oracle/block.py), through the C
ABI, and of the three steps chained (prologue, scan, gated norm).

bfloat16 outputs are compared with gpu_util.rel_err at 2e-2; dt (fp32) at
1e-5.  At the Mamba-2 2.7B shape the oracle runs on token windows (the
convolution looks W - 1 tokens back, so a window's outputs from its W-th token
on are exact) and on sampled tokens of the norm.  Every case prints its name
and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
from gpu_util import TOL, announce, rel_err, to_np

pytestmark = pytest.mark.gpu

dev = "cuda"


def _t(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev, dtype=dtype)


def _prologue_gpu(b, H, P, G, N):
    import selective_state_space_chunk_amd as ssd
    out = ssd.ssd_block_prologue(_t(b["zxbcdt"], torch.bfloat16), _t(b["conv_w"]), _t(b["conv_b"]),
                                 _t(b["dt_bias"]), H, P, G, N)
    torch.cuda.synchronize()
    return out


# (name, B, L, H, P, G, N, W)
PRO = [
    ("ragged_rows_w4", 2, 150, 8, 64, 1, 128, 4),
    ("groups_w3", 1, 64, 8, 64, 2, 64, 3),
    ("short_rows_w4", 3, 5, 8, 16, 1, 16, 4),
    ("w2", 1, 70, 8, 32, 1, 32, 2),
    ("w1", 1, 33, 8, 32, 1, 32, 1),
    # three 128-token tiles, the last ragged: the convolution's history crosses tile edges
    ("tiles_ragged_w4", 2, 300, 8, 64, 1, 64, 4),
]


@pytest.mark.parametrize("case", PRO, ids=[c[0] for c in PRO])
def test_prologue_matches_oracle(case):
    name, B, L, H, P, G, N, W = case
    b = si.make_block_inputs(B, L, H, P, G, N, W, seed=5100 + L)
    ref = oracle.block_prologue(b["zxbcdt"], b["conv_w"], b["conv_b"], b["dt_bias"], H, P, G, N)
    announce(f"prologue {name}: B{B} L{L} H{H} P{P} G{G} N{N} W{W}")
    got = _prologue_gpu(b, H, P, G, N)
    for k in ("x", "Bm", "Cm"):
        e = rel_err(to_np(got[k]), ref[k])
        print(f"    {k}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)
    e = rel_err(to_np(got["dt"]), ref["dt"])
    assert e <= 1e-5, ("dt", e)
    assert got["z"].shape == (B, L, H * P)


# (name, T, D, ngroups, center, bias, strided z)
NORM = [
    ("group_norm_one_group", 37, 512, 1, True, True, False),
    ("group_norm_eight_groups", 20, 1024, 8, True, False, True),
    ("rms_four_groups", 33, 256, 4, False, True, True),
    ("rms_widest", 9, 8192, 2, False, False, False),
    ("odd_width", 5, 200, 1, True, True, False),
]


@pytest.mark.parametrize("case", NORM, ids=[c[0] for c in NORM])
def test_gated_norm_matches_oracle(case):
    import selective_state_space_chunk_amd as ssd
    name, T, D, ng, center, with_bias, strided = case
    rng = np.random.default_rng(5200 + D)
    y = si.round_bf16(rng.standard_normal((T, D)))
    zfull = si.round_bf16(rng.standard_normal((T, D + 40)))
    z = zfull[:, 8:8 + D] if strided else zfull[:, :D]
    w = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(D)).astype(np.float32) if with_bias else None
    ref = oracle.gated_norm(y, z, w, bias, ng, 1e-5, center)
    announce(f"gated norm {name}: T{T} D{D} groups {ng} center={center} bias={with_bias} strided z={strided}")
    zt = _t(zfull, torch.bfloat16)[:, 8:8 + D] if strided else _t(z, torch.bfloat16)
    out = ssd.ssd_gated_norm(_t(y, torch.bfloat16), zt, _t(w), None if bias is None else _t(bias), ng, 1e-5, center)
    torch.cuda.synchronize()
    e = rel_err(to_np(out), ref)
    print(f"    out: {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e


def test_block_steps_chained():
    # The three steps chained on the GPU (prologue -> scan -> gated norm)
    # against a chain that runs only the oracle: the oracle prologue, its x,
    # Bm, Cm rounded to bfloat16 and dt to float32 as the GPU stores them, the
    # oracle scan, its y rounded to bfloat16, the oracle norm.  No value of the
    # GPU chain enters the reference.
    import selective_state_space_chunk_amd as ssd
    B, L, H, P, G, N, W = 2, 300, 8, 64, 1, 128, 4
    b = si.make_block_inputs(B, L, H, P, G, N, W, seed=5301)
    A = -np.exp(np.random.default_rng(5302).uniform(-1.0, 1.5, H)).astype(np.float32)
    D = np.random.default_rng(5303).standard_normal(H).astype(np.float32)
    pro = oracle.block_prologue(b["zxbcdt"], b["conv_w"], b["conv_b"], b["dt_bias"], H, P, G, N)
    xr, Br, Cr = (si.round_bf16(pro[k]).astype(np.float64) for k in ("x", "Bm", "Cm"))
    dtr = pro["dt"].astype(np.float32).astype(np.float64)
    y_ref, _ = oracle.recurrence(xr, dtr, A.astype(np.float64), Br, Cr, D.astype(np.float64), None)
    out_ref = oracle.gated_norm(si.round_bf16(y_ref).reshape(B * L, H * P), pro["z"].reshape(B * L, H * P),
                                b["norm_w"], b["norm_b"], 1, 1e-5, True)
    announce(f"block chain: prologue, scan, gated norm; B{B} L{L} H{H} P{P} N{N}")
    g = _prologue_gpu(b, H, P, G, N)
    for k in ("x", "Bm", "Cm"):
        e = rel_err(to_np(g[k]), pro[k])
        print(f"    prologue {k}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)
    e = rel_err(to_np(g["dt"]), pro["dt"])
    assert e <= 1e-5, ("dt", e)
    y, _ = ssd.ssd_chunk_scan_fwd(g["x"], g["dt"], _t(A), g["Bm"], g["Cm"], _t(D), None)
    out = ssd.ssd_gated_norm(y, g["z"], _t(b["norm_w"]), _t(b["norm_b"]), 1, 1e-5, True)
    torch.cuda.synchronize()
    e = rel_err(to_np(y), y_ref)
    print(f"    scan y: {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e
    e = rel_err(to_np(out).reshape(B * L, H * P), out_ref)
    print(f"    out: {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e


def test_full_size_windows():
    import selective_state_space_chunk_amd as ssd
    B, L, H, P, G, N, W = 4, 4096, 80, 64, 1, 128, 4
    b = si.make_block_inputs(B, L, H, P, G, N, W, seed=5401)
    announce(f"block steps at full size: B{B} L{L} H{H} P{P} N{N} W{W}")
    g = _prologue_gpu(b, H, P, G, N)
    for t0, t1 in ((0, 70), (2040, 2110), (4026, 4096)):
        s0 = max(0, t0 - (W - 1))
        ref = oracle.block_prologue(b["zxbcdt"][:, s0:t1], b["conv_w"], b["conv_b"], b["dt_bias"], H, P, G, N)
        k0 = t0 - s0
        for k in ("x", "Bm", "Cm", "dt"):
            e = rel_err(to_np(g[k][:, t0:t1]), ref[k][:, k0:])
            assert e <= (1e-5 if k == "dt" else TOL["bf16"]), (t0, k, e)
    y = _t(b["y"], torch.bfloat16)
    out = ssd.ssd_gated_norm(y, g["z"], _t(b["norm_w"]), _t(b["norm_b"]), 1, 1e-5, True)
    torch.cuda.synchronize()
    T = B * L
    idx = np.arange(0, T, 97)
    z = b["zxbcdt"].reshape(T, -1)[idx, :H * P]
    ref = oracle.gated_norm(b["y"].reshape(T, H * P)[idx], z, b["norm_w"], b["norm_b"], 1, 1e-5, True)
    e = rel_err(to_np(out).reshape(T, H * P)[idx], ref)
    print(f"    norm sampled: {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e


def test_uncovered_shapes_are_rejected():
    import selective_state_space_chunk_amd as ssd
    announce("block steps: W = 5 and D = 8200 are not covered")
    b = si.make_block_inputs(1, 10, 8, 32, 1, 32, 5, seed=5501)
    with pytest.raises(ssd.SSDError) as ei:
        _prologue_gpu(b, 8, 32, 1, 32)
    assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED
    y = torch.zeros((3, 8200), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ssd.SSDError) as ei:
        ssd.ssd_gated_norm(y, y, torch.ones(8200, device=dev))
    assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED


def test_130m_shape_windows():
    # the Mamba-2 130M layer shape: H 24 (HP 1536), N 128, W 4; norm in 4 groups, RMS
    import selective_state_space_chunk_amd as ssd
    B, L, H, P, G, N, W = 8, 2048, 24, 64, 1, 128, 4
    b = si.make_block_inputs(B, L, H, P, G, N, W, seed=5601)
    announce(f"block steps at the 130M shape: B{B} L{L} H{H} P{P} N{N} W{W}")
    g = _prologue_gpu(b, H, P, G, N)
    for t0, t1 in ((0, 40), (1000, 1040), (2008, 2048)):
        s0 = max(0, t0 - (W - 1))
        ref = oracle.block_prologue(b["zxbcdt"][:, s0:t1], b["conv_w"], b["conv_b"], b["dt_bias"], H, P, G, N)
        for k in ("x", "Bm", "Cm", "dt"):
            e = rel_err(to_np(g[k][:, t0:t1]), ref[k][:, t0 - s0:])
            assert e <= (1e-5 if k == "dt" else TOL["bf16"]), (t0, k, e)
    out = ssd.ssd_gated_norm(_t(b["y"], torch.bfloat16), g["z"], _t(b["norm_w"]), None, 4, 1e-5, False)
    torch.cuda.synchronize()
    T = B * L
    idx = np.arange(0, T, 61)
    z = b["zxbcdt"].reshape(T, -1)[idx, :H * P]
    ref = oracle.gated_norm(b["y"].reshape(T, H * P)[idx], z, b["norm_w"], None, 4, 1e-5, False)
    e = rel_err(to_np(out).reshape(T, H * P)[idx], ref)
    print(f"    norm sampled: {e:.3e}", flush=True)
    assert e <= TOL["bf16"], e
