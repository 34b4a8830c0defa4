"""Pins of the block prologue / gated-norm oracle (oracle/block.py) against
library routines and closed forms:

* the causal depthwise convolution equals numpy's full convolution of each
  channel with the reversed taps, cut to the first L outputs; SiLU is checked
  through scipy's logistic function;
* a unit tap on the newest token makes the convolution the identity plus bias;
* softplus: softplus(0) = ln 2 and softplus(v) - softplus(-v) = v;
* the split hands every slice of the projection to the right output;
* the centred norm equals torch's group_norm and the uncentred one torch's
  rms_norm on each group (CPU, float64); a large constant gate input scales y
  uniformly (SiLU(z) = z there), which leaves the plain norm of y; without
  eps the result does not change when y is scaled.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle.block import block_prologue, gated_norm, softplus


def _proj(seed, B, L, H, P, G, N, W):
    rng = np.random.default_rng(seed)
    C = H * P + 2 * G * N
    return (rng.standard_normal((B, L, 2 * H * P + 2 * G * N + H)), rng.standard_normal((C, W)) / 2,
            rng.standard_normal(C) / 4, rng.standard_normal(H))


def test_conv_is_numpy_convolution_and_silu():
    B, L, H, P, G, N, W = 2, 11, 2, 3, 1, 4, 4
    v, w, cb, db = _proj(1, B, L, H, P, G, N, W)
    out = block_prologue(v, w, cb, db, H, P, G, N)
    d, gn = H * P, G * N
    act = np.concatenate([out["x"].reshape(B, L, d), out["Bm"].reshape(B, L, gn), out["Cm"].reshape(B, L, gn)], axis=2)
    for b in range(B):
        for c in range(d + 2 * gn):
            conv = np.convolve(v[b, :, d + c], w[c][::-1])[:L] + cb[c]
            np.testing.assert_allclose(act[b, :, c], conv * expit(conv), rtol=1e-12, atol=1e-12)


def test_unit_tap_is_identity_plus_bias():
    B, L, H, P, G, N, W = 1, 6, 2, 2, 1, 2, 4
    v, w, cb, db = _proj(2, B, L, H, P, G, N, W)
    w[:] = 0.0
    w[:, W - 1] = 1.0
    out = block_prologue(v, w, cb, db, H, P, G, N)
    pre = v[0, :, H * P:H * P + H * P] + cb[:H * P]
    np.testing.assert_allclose(out["x"].reshape(L, H * P), pre * expit(pre), rtol=1e-12)


def test_softplus_closed_forms():
    assert softplus(np.array(0.0)) == pytest.approx(np.log(2.0), rel=1e-15)
    v = np.linspace(-30, 30, 61)
    np.testing.assert_allclose(softplus(v) - softplus(-v), v, rtol=1e-12, atol=1e-12)


def test_split_routes_every_slice():
    B, L, H, P, G, N, W = 1, 3, 2, 2, 2, 3, 1
    d, gn = H * P, G * N
    v = np.arange(B * L * (2 * d + 2 * gn + H), dtype=np.float64).reshape(B, L, -1) / 100.0
    out = block_prologue(v, np.ones((d + 2 * gn, 1)), np.zeros(d + 2 * gn), np.zeros(H), H, P, G, N)
    np.testing.assert_array_equal(out["z"], v[:, :, :d])
    s = lambda a: a * expit(a)
    np.testing.assert_allclose(out["x"].reshape(B, L, d), s(v[:, :, d:2 * d]), rtol=1e-14)
    np.testing.assert_allclose(out["Bm"].reshape(B, L, gn), s(v[:, :, 2 * d:2 * d + gn]), rtol=1e-14)
    np.testing.assert_allclose(out["Cm"].reshape(B, L, gn), s(v[:, :, 2 * d + gn:2 * d + 2 * gn]), rtol=1e-14)
    np.testing.assert_allclose(out["dt"], softplus(v[:, :, 2 * d + 2 * gn:]), rtol=1e-14)


@pytest.mark.parametrize("ngroups", [1, 4])
def test_norms_match_torch(ngroups):
    rng = np.random.default_rng(3)
    T, D = 7, 32
    y, z = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    wt, bs = rng.standard_normal(D), rng.standard_normal(D)
    gated = torch.from_numpy(y * (z * expit(z)))
    want = torch.nn.functional.group_norm(gated, ngroups, torch.from_numpy(wt), torch.from_numpy(bs), eps=1e-5)
    np.testing.assert_allclose(gated_norm(y, z, wt, bs, ngroups, 1e-5, True), want.numpy(), rtol=1e-10, atol=1e-10)
    r = torch.nn.functional.rms_norm(gated.reshape(T, ngroups, D // ngroups), (D // ngroups,), eps=1e-5)
    np.testing.assert_allclose(gated_norm(y, z, wt, None, ngroups, 1e-5, False), r.reshape(T, D).numpy() * wt,
                               rtol=1e-10, atol=1e-10)


def test_open_gate_and_scale_invariance():
    rng = np.random.default_rng(4)
    T, D = 5, 24
    y = rng.standard_normal((T, D))
    wt = rng.standard_normal(D)
    open_gate = gated_norm(y, np.full((T, D), 60.0), wt, None, 2, 0.0, False)
    g = y.reshape(T, 2, 12)
    np.testing.assert_allclose(open_gate, (g / np.sqrt((g * g).mean(axis=2, keepdims=True))).reshape(T, D) * wt,
                               rtol=1e-12)
    z = rng.standard_normal((T, D))
    for center in (True, False):
        np.testing.assert_allclose(gated_norm(3.5 * y, z, wt, None, 3, 0.0, center),
                                   gated_norm(y, z, wt, None, 3, 0.0, center), rtol=1e-12, atol=1e-12)
