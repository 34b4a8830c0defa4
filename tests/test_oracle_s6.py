"""Pins of the selective-scan oracle (oracle/s6.py):

* the pages' gating case ("Mamba" reading notes, Theorem 1): N = 1, A = -1,
  B = 1 and dt = softplus(z) turn the zero-order-hold recurrence into
  h_t = (1 - g_t) h_{t-1} + g_t x_t with g_t = sigmoid(z_t), exactly;
* with the simple input term and one decay per channel, the scan is the SSD
  recurrence with one-wide heads (oracle.recurrence, P = 1, a channel per head);
* a brute-force double sum over (t, s) with per-state decays (tiny sizes), for
  both input terms;
* zero-order hold tends to the simple input term as A -> 0, and A = 0 takes
  the limit itself.
"""
import numpy as np
from scipy.special import expit

import oracle
from oracle.s6 import selective_scan


def _inputs(seed, B, L, Dch, N, G):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((B, L, Dch)),
                dt=np.log1p(np.exp(rng.standard_normal((B, L, Dch)) - 1.0)),
                A=-np.exp(rng.uniform(-1.0, 1.0, (Dch, N))),
                Bm=rng.standard_normal((B, L, G, N)), Cm=rng.standard_normal((B, L, G, N)),
                D=rng.standard_normal(Dch), init=rng.standard_normal((B, Dch, N)) * 0.3)


def test_gating_case_of_theorem_one():
    rng = np.random.default_rng(1)
    L = 25
    z = rng.standard_normal((1, L, 1)) * 2
    x = rng.standard_normal((1, L, 1))
    dt = np.logaddexp(0.0, z)
    ones = np.ones((1, L, 1, 1))
    y, fin = selective_scan(x, dt, -np.ones((1, 1)), ones, ones, None, np.full((1, 1, 1), 0.4), zoh=True)
    g = expit(z[0, :, 0])
    h = 0.4
    for t in range(L):
        h = (1 - g[t]) * h + g[t] * x[0, t, 0]
        assert abs(y[0, t, 0] - h) <= 1e-12 * max(1.0, abs(h))
    assert abs(fin[0, 0, 0] - h) <= 1e-12


def test_simple_term_with_one_decay_is_the_ssd_recurrence():
    B, L, Dch, N, G = 2, 30, 6, 5, 3
    d = _inputs(2, B, L, Dch, N, G)
    A1 = -np.exp(np.random.default_rng(3).uniform(-1, 1, Dch))
    y, fin = selective_scan(d["x"], d["dt"], np.repeat(A1[:, None], N, axis=1), d["Bm"], d["Cm"], d["D"], d["init"],
                            zoh=False)
    ys, fs = oracle.recurrence(d["x"][..., None], d["dt"], A1, d["Bm"], d["Cm"], d["D"], d["init"][:, :, None, :])
    np.testing.assert_allclose(y, ys[..., 0], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(fin, fs[:, :, 0, :], rtol=1e-11, atol=1e-11)


def test_brute_force_double_sum():
    B, L, Dch, N, G = 1, 9, 4, 3, 2
    d = _inputs(4, B, L, Dch, N, G)
    for zoh in (True, False):
        y, _ = selective_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], None, zoh=zoh)
        for c in range(Dch):
            g = c // (Dch // G)
            for t in range(L):
                acc = d["D"][c] * d["x"][0, t, c]
                for s in range(t + 1):
                    for n in range(N):
                        An, ds = d["A"][c, n], d["dt"][0, s, c]
                        decay = np.exp(An * sum(d["dt"][0, r, c] for r in range(s + 1, t + 1)))
                        bbar = (np.exp(ds * An) - 1.0) / An if zoh else ds
                        acc += d["Cm"][0, t, g, n] * decay * bbar * d["Bm"][0, s, g, n] * d["x"][0, s, c]
                assert abs(y[0, t, c] - acc) <= 1e-10 * max(1.0, abs(acc)), (zoh, c, t)


def test_zero_order_hold_limit_at_zero_decay():
    B, L, Dch, N, G = 1, 12, 3, 4, 1
    d = _inputs(5, B, L, Dch, N, G)
    simple, _ = selective_scan(d["x"], d["dt"], np.zeros((Dch, N)), d["Bm"], d["Cm"], d["D"], d["init"], zoh=False)
    at_zero, _ = selective_scan(d["x"], d["dt"], np.zeros((Dch, N)), d["Bm"], d["Cm"], d["D"], d["init"], zoh=True)
    near, _ = selective_scan(d["x"], d["dt"], np.full((Dch, N), -1e-9), d["Bm"], d["Cm"], d["D"], d["init"], zoh=True)
    np.testing.assert_array_equal(at_zero, simple)
    np.testing.assert_allclose(near, simple, rtol=1e-7, atol=1e-7)
