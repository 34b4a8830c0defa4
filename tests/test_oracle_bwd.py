"""Pins of the fp64 gradient oracle (oracle/backward.py) against what the
mathematics fixes, independently of its own code:

* central finite differences of the forward recurrence oracle, for every
  input (grouped heads, initial state, a gradient on the final state);
* exact adjointness in x and in the initial state (y and the final state are
  linear in them, so <dy, y(x+v) - y(x)> = <dx, v> up to rounding);
* closed forms with no decay (A = 0, dt = 1), where the scan is causal linear
  attention: y = tril(Cm Bm^T) x + D x, whose gradients are matrix products,
  and dA = sum_{s<t} (t - s) (dy_t . x_s)(Cm_t . Bm_s).
"""
import numpy as np
import pytest

import oracle
from oracle.backward import recurrence_bwd


def _inputs(seed, B, L, H, P, G, N, init=True):
    rng = np.random.default_rng(seed)
    d = dict(x=rng.standard_normal((B, L, H, P)),
             dt=np.log1p(np.exp(rng.standard_normal((B, L, H)) - 1.0)),
             A=-np.exp(rng.uniform(0.0, 1.5, H)),
             Bm=rng.standard_normal((B, L, G, N)) / 2,
             Cm=rng.standard_normal((B, L, G, N)) / 2,
             D=rng.standard_normal(H),
             init=rng.standard_normal((B, H, P, N)) * 0.3 if init else None)
    dy = rng.standard_normal((B, L, H, P))
    dfinal = rng.standard_normal((B, H, P, N))
    return d, dy, dfinal


def _objective(d, dy, dfinal):
    y, f = oracle.recurrence(**d)
    j = float(np.sum(dy * y))
    if dfinal is not None:
        j += float(np.sum(dfinal * f))
    return j


NAMES = {"x": "dx", "dt": "ddt", "A": "dA", "Bm": "dBm", "Cm": "dCm", "D": "dD", "init": "dinit"}


@pytest.mark.parametrize("shape,with_dfinal", [((2, 7, 4, 3, 2, 5), True), ((1, 9, 2, 2, 1, 3), False)])
def test_gradients_match_central_differences(shape, with_dfinal):
    B, L, H, P, G, N = shape
    d, dy, dfinal = _inputs(11 + L, B, L, H, P, G, N)
    if not with_dfinal:
        dfinal = None
    g = recurrence_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], dy, dfinal)
    eps = 1e-6
    for name, gname in NAMES.items():
        v = d[name]
        fd = np.zeros_like(v)
        for idx in np.ndindex(v.shape):
            up, dn = dict(d), dict(d)
            up[name] = v.copy()
            up[name][idx] += eps
            dn[name] = v.copy()
            dn[name][idx] -= eps
            fd[idx] = (_objective(up, dy, dfinal) - _objective(dn, dy, dfinal)) / (2 * eps)
        err = np.max(np.abs(fd - g[gname])) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)


def test_adjoint_is_exact_in_x_and_initial_state():
    d, dy, dfinal = _inputs(3, 2, 12, 3, 4, 1, 6)
    g = recurrence_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], dy, dfinal)
    rng = np.random.default_rng(4)
    base = _objective(d, dy, dfinal)
    for name in ("x", "init"):
        v = rng.standard_normal(d[name].shape)
        moved = dict(d)
        moved[name] = d[name] + v
        lhs = _objective(moved, dy, dfinal) - base
        rhs = float(np.sum(g[NAMES[name]] * v))
        assert abs(lhs - rhs) <= 1e-11 * max(1.0, abs(rhs)), (name, lhs, rhs)


def test_no_decay_gradients_are_the_linear_attention_ones():
    # one head, one group, unit steps, no decay, zero initial state
    rng = np.random.default_rng(9)
    L, P, N = 10, 3, 4
    x = rng.standard_normal((1, L, 1, P))
    Bm = rng.standard_normal((1, L, 1, N))
    Cm = rng.standard_normal((1, L, 1, N))
    dy = rng.standard_normal((1, L, 1, P))
    D = np.array([0.7])
    g = recurrence_bwd(x, np.ones((1, L, 1)), np.zeros(1), Bm, Cm, D, None, dy, None)
    X, Y, Bq, Cq = x[0, :, 0], dy[0, :, 0], Bm[0, :, 0], Cm[0, :, 0]
    M = np.tril(Cq @ Bq.T)                       # y = M X + D X
    K = np.tril(Y @ X.T)                         # K[t, s] = dy_t . x_s for s <= t
    np.testing.assert_allclose(g["dx"][0, :, 0], M.T @ Y + D[0] * Y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dCm"][0, :, 0], K @ Bq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dBm"][0, :, 0], K.T @ Cq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dD"], [np.sum(Y * X)], rtol=1e-12)
    KC = K * (Cq @ Bq.T)                         # (dy_t . x_s)(Cm_t . Bm_s), s <= t
    np.testing.assert_allclose(g["ddt"][0, :, 0], KC.sum(axis=0), rtol=1e-12, atol=1e-12)
    t_minus_s = np.subtract.outer(np.arange(L), np.arange(L))
    np.testing.assert_allclose(g["dA"], [np.sum(KC * t_minus_s)], rtol=1e-12)
