"""GPU parity of ssd_chunk_scan_bwd against the fp64 gradient oracle, through
the C ABI.

The oracle (oracle/backward.py, the adjoint of the token recurrence) runs on
exactly the values the GPU receives.  Every gradient is compared with the
metric of gpu_util.rel_err (max |got - ref| / max |ref| over the tensor) at the
bfloat16 limit, 2e-2.  Every case prints its name and shape before it touches
the GPU.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, rel_err, to_device, to_np

from oracle.backward import recurrence_bwd

pytestmark = pytest.mark.gpu

GRADS = ("dx", "ddt", "dA", "dBm", "dCm", "dD", "dinit")


def oracle_grads(d, g):
    f = si.as_f64(d)
    gf = si.as_f64(g)
    return recurrence_bwd(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], gf["dy"], gf["dfinal"])


def gpu_grads(dd, dg, chunk=256):
    import selective_state_space_chunk_amd as ssd
    out = ssd.ssd_chunk_scan_bwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], dd["init"],
                                 dg["dy"], dg["dfinal"], chunk)
    torch.cuda.synchronize()
    return out


def grad_device(g):
    return {"dy": torch.from_numpy(g["dy"]).to("cuda", dtype=torch.bfloat16),
            "dfinal": None if g["dfinal"] is None else torch.from_numpy(g["dfinal"]).to("cuda")}


# (name, B, L, H, N, G, init, dfinal, regime)
CASES = [
    ("one_block", 1, 64, 2, 128, 1, True, True, "default"),
    ("ragged_three_blocks", 2, 3 * 64 + 17, 4, 128, 1, True, True, "default"),
    ("groups_n64", 2, 150, 4, 64, 2, True, False, "long_memory"),
    ("no_init_no_dfinal", 1, 200, 3, 128, 3, False, False, "default"),
    ("one_token", 2, 1, 2, 128, 1, True, True, "default"),
    ("long_memory_many_blocks", 1, 1100, 2, 128, 1, True, True, "long_memory"),
    ("no_decay", 1, 260, 2, 64, 1, True, True, "no_decay"),
    # the head counts per group of the layer shapes: dBm and dCm are summed over
    # every head of a group in matrix-core accumulators, dA and dD over tokens
    ("eighty_heads_one_group", 1, 300, 80, 128, 1, True, True, "default"),
    ("twenty_four_heads_one_group", 2, 140, 24, 128, 1, True, False, "default"),
    ("five_heads_one_group", 2, 200, 5, 128, 1, True, True, "default"),
    ("three_heads_per_group", 1, 180, 6, 64, 2, True, True, "long_memory"),
    # the dLambda / ddt tails run once per batch of eight heads: a full batch
    # followed by a partial one
    ("thirteen_heads_one_group", 1, 150, 13, 128, 1, True, True, "default"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, B, L, H, N, G, init, dfin, regime = case
    d = si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=init, seed=3100 + L + H, regime=regime)
    g = si.make_grad_inputs(B, L, H, 64, N, dtype="bf16", dfinal=dfin, seed=3200 + L)
    ref = oracle_grads(d, g)
    announce(f"bwd {name}: B{B} L{L} H{H} P64 N{N} G{G} init={init} dfinal={dfin} {regime}")
    got = gpu_grads(to_device(d, "bf16"), grad_device(g))
    for k in GRADS:
        e = rel_err(to_np(got[k]), ref[k])
        print(f"    {k}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)


# heads of 128 channels: each is taken as two heads of 64 sharing dt, A and D,
# whose ddt, dA and dD are the sums over the two halves
# (name, B, L, H, N, G, init, dfinal, regime)
CASES_P128 = [
    ("p128_one_block", 1, 64, 2, 128, 1, True, True, "default"),
    ("p128_ragged", 2, 3 * 64 + 17, 3, 128, 1, True, True, "default"),
    ("p128_groups_n64", 2, 150, 4, 64, 2, False, True, "long_memory"),
    ("p128_forty_heads_one_group", 1, 260, 40, 128, 1, True, False, "default"),
    # ten heads of 64: a batch of four heads of 128, then a batch of one
    ("p128_five_heads_one_group", 1, 150, 5, 128, 1, True, True, "default"),
]


@pytest.mark.parametrize("case", CASES_P128, ids=[c[0] for c in CASES_P128])
def test_backward_head_dim_128(case):
    name, B, L, H, N, G, init, dfin, regime = case
    d = si.make_scan_inputs(B, L, H, 128, N, G, dtype="bf16", init=init, seed=3600 + L + H, regime=regime)
    g = si.make_grad_inputs(B, L, H, 128, N, dtype="bf16", dfinal=dfin, seed=3700 + L)
    ref = oracle_grads(d, g)
    announce(f"bwd {name}: B{B} L{L} H{H} P128 N{N} G{G} init={init} dfinal={dfin} {regime}")
    got = gpu_grads(to_device(d, "bf16"), grad_device(g))
    for k in GRADS:
        e = rel_err(to_np(got[k]), ref[k])
        print(f"    {k}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)


def test_backward_is_deterministic():
    d = si.make_scan_inputs(1, 300, 4, 64, 128, 1, dtype="bf16", init=True, seed=3301)
    g = si.make_grad_inputs(1, 300, 4, 64, 128, dtype="bf16", seed=3302)
    dd, dg = to_device(d, "bf16"), grad_device(g)
    announce("bwd determinism: B1 L300 H4 N128, two calls")
    a = gpu_grads(dd, dg)
    b = gpu_grads(dd, dg)
    for k in GRADS:
        assert torch.equal(a[k], b[k]), k


def test_backward_without_tokens():
    import selective_state_space_chunk_amd as ssd
    H, N = 3, 64
    dfinal = torch.randn(2, H, 64, N, device="cuda")
    x = torch.empty((2, 0, H, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((2, 0, H), device="cuda")
    Bm = torch.empty((2, 0, 1, N), dtype=torch.bfloat16, device="cuda")
    announce("bwd with L = 0")
    out = ssd.ssd_chunk_scan_bwd(x, dt, torch.full((H,), -1.0, device="cuda"), Bm, Bm.clone(),
                                 torch.ones(H, device="cuda"), None, torch.empty_like(x), dfinal)
    torch.cuda.synchronize()
    assert torch.equal(out["dinit"], dfinal)
    assert torch.count_nonzero(out["dA"]) == 0 and torch.count_nonzero(out["dD"]) == 0


def test_backward_rejects_uncovered_shapes():
    import selective_state_space_chunk_amd as ssd
    d = si.make_scan_inputs(1, 70, 2, 32, 64, 1, dtype="bf16", seed=3303)
    g = si.make_grad_inputs(1, 70, 2, 32, 64, dtype="bf16", seed=3304)
    dd, dg = to_device(d, "bf16"), grad_device(g)
    announce("bwd P=32 is not covered")
    with pytest.raises(ssd.SSDError) as ei:
        gpu_grads(dd, dg)
    assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED


def test_backward_at_the_130m_shape_sampled_heads():
    # the Mamba-2 130M layer shape: B 8, L 2048, H 24; the oracle on three (batch, head) pairs
    B, L, H, N = 8, 2048, 24, 128
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=3401)
    g = si.make_grad_inputs(B, L, H, 64, N, dtype="bf16", seed=3402)
    announce(f"bwd at the 130M shape: B{B} L{L} H{H} N{N}, sampled heads")
    got = gpu_grads(to_device(d, "bf16"), grad_device(g))
    f, gf = si.as_f64(d), si.as_f64(g)
    for b, h in ((0, 0), (3, 11), (7, 23)):
        sl = lambda a, ax=2: np.take(a[b:b + 1], [h], axis=ax)
        ref = recurrence_bwd(sl(f["x"]), sl(f["dt"]), f["A"][[h]], f["Bm"][b:b + 1], f["Cm"][b:b + 1], f["D"][[h]],
                             sl(f["init"], 1), sl(gf["dy"]), sl(gf["dfinal"], 1))
        for k, gk in (("dx", got["dx"][b:b + 1, :, h:h + 1]), ("ddt", got["ddt"][b:b + 1, :, h:h + 1]),
                      ("dinit", got["dinit"][b:b + 1, h:h + 1])):
            e = rel_err(to_np(gk), ref[k])
            print(f"    b{b} h{h} {k}: {e:.3e}", flush=True)
            assert e <= TOL["bf16"], (b, h, k, e)


def test_backward_at_the_2p7b_shape_sampled_heads():
    # the Mamba-2 2.7B layer shape the bench times: B 4, L 4096, H 80, N 128,
    # one group, a random initial state.  The oracle runs on sampled (batch,
    # head) pairs for dx, ddt and dinit, and on every batch row of two heads
    # for dA and dD (summed over batch rows and tokens).  dBm and dCm sum over
    # all 80 heads; they are compared at 80 heads per group in
    # eighty_heads_one_group above.
    B, L, H, N = 4, 4096, 80, 128
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=3501)
    g = si.make_grad_inputs(B, L, H, 64, N, dtype="bf16", seed=3502)
    announce(f"bwd at the 2.7B shape: B{B} L{L} H{H} N{N}, sampled heads")
    got = gpu_grads(to_device(d, "bf16"), grad_device(g))
    f, gf = si.as_f64(d), si.as_f64(g)
    for b, h in ((0, 0), (2, 41), (3, 79)):
        sl = lambda a, ax=2: np.take(a[b:b + 1], [h], axis=ax)
        ref = recurrence_bwd(sl(f["x"]), sl(f["dt"]), f["A"][[h]], f["Bm"][b:b + 1], f["Cm"][b:b + 1], f["D"][[h]],
                             sl(f["init"], 1), sl(gf["dy"]), sl(gf["dfinal"], 1))
        for k, gk in (("dx", got["dx"][b:b + 1, :, h:h + 1]), ("ddt", got["ddt"][b:b + 1, :, h:h + 1]),
                      ("dinit", got["dinit"][b:b + 1, h:h + 1])):
            e = rel_err(to_np(gk), ref[k])
            print(f"    b{b} h{h} {k}: {e:.3e}", flush=True)
            assert e <= TOL["bf16"], (b, h, k, e)
    # dA and dD of the sampled heads as one tensor each (the metric's scale is
    # the largest magnitude over the sampled heads)
    heads = [7, 66]
    sl = lambda a, ax=2: np.take(a, heads, axis=ax)
    ref = recurrence_bwd(sl(f["x"]), sl(f["dt"]), f["A"][heads], f["Bm"], f["Cm"], f["D"][heads],
                         sl(f["init"], 1), sl(gf["dy"]), sl(gf["dfinal"], 1))
    for k in ("dA", "dD"):
        e = rel_err(to_np(got[k][heads]), ref[k])
        print(f"    heads {heads} {k}: {e:.3e}", flush=True)
        assert e <= TOL["bf16"], (k, e)
