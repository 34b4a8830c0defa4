"""Pins of the packed-sequence oracle (oracle/varlen.py) against what the
mathematics fixes, independently of how it cuts the rows:

* a state reset is the same as a decay of zero at the first token of every
  later sequence, so a token recurrence written here with a_t = 0 at those
  tokens must agree on every output and final state;
* with no boundaries the result is the plain recurrence's, bit for bit;
* the first token of every later sequence sees no earlier token:
  y_t = dt_t (Cm_t . Bm_t) x_t + D x_t, a closed form, and the same holds for
  every token when every token is its own sequence;
* outputs of one sequence do not change when another sequence's inputs do;
* the generator's rows are non-decreasing runs that start at 0.
"""
import numpy as np
import pytest

import oracle
import ssd_inputs as si
from oracle.varlen import recurrence_varlen, run_bounds


def _inputs(seed, B, L, H, P, G, N, init=True):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((B, L, H, P)),
                dt=np.log1p(np.exp(rng.standard_normal((B, L, H)) - 1.0)),
                A=-np.exp(rng.uniform(-1.0, 1.0, H)),
                Bm=rng.standard_normal((B, L, G, N)) / 2,
                Cm=rng.standard_normal((B, L, G, N)) / 2,
                D=rng.standard_normal(H),
                init=rng.standard_normal((B, H, P, N)) if init else None)


def _reset_recurrence(d, seq):
    """S_t = a_t S_{t-1} + dt_t x_t Bm_t^T with a_t = 0 where a new sequence
    starts, y_t = S_t Cm_t + D x_t; one loop per (batch, head)."""
    x, dt, A, Bm, Cm, D, init = (d[k] for k in ("x", "dt", "A", "Bm", "Cm", "D", "init"))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y = np.zeros_like(x)
    fin = np.zeros((Bsz, H, P, N))
    for b in range(Bsz):
        for h in range(H):
            g = h // (H // G)
            S = np.zeros((P, N)) if init is None else init[b, h].copy()
            for t in range(L):
                a = 0.0 if (t > 0 and seq[b, t] != seq[b, t - 1]) else np.exp(dt[b, t, h] * A[h])
                S = a * S + dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, g])
                y[b, t, h] = S @ Cm[b, t, g] + D[h] * x[b, t, h]
            fin[b, h] = S
    return y, fin


@pytest.mark.parametrize("lengths", [[[3, 5, 1, 7]], [[1, 1, 14]], [[16]], [[9, 7], [2, 2, 2, 10]]])
def test_matches_reset_recurrence(lengths):
    B, L = len(lengths), 16
    d = _inputs(5 + B, B, L, 3, 4, 3, 5)
    seq = si.make_seq_idx(B, L, lengths=lengths)
    y, f = recurrence_varlen(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], seq)
    yr, fr = _reset_recurrence(d, seq)
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f, fr, rtol=1e-12, atol=1e-12)


def test_no_boundary_is_the_plain_recurrence():
    d = _inputs(7, 2, 40, 2, 3, 1, 4)
    seq = np.zeros((2, 40), dtype=np.int32)
    y, f = recurrence_varlen(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], seq)
    y0, f0 = oracle.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"])
    assert np.array_equal(y, y0) and np.array_equal(f, f0)


def test_first_token_of_a_sequence_sees_nothing_earlier():
    B, L, H, P, G, N = 1, 30, 2, 3, 1, 4
    d = _inputs(8, B, L, H, P, G, N)
    seq = si.make_seq_idx(B, L, lengths=[[11, 6, 13]])
    y, _ = recurrence_varlen(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], seq)
    for t in (11, 17):
        for h in range(H):
            cb = float(d["Cm"][0, t, 0] @ d["Bm"][0, t, 0])
            want = (d["dt"][0, t, h] * cb + d["D"][h]) * d["x"][0, t, h]
            np.testing.assert_allclose(y[0, t, h], want, rtol=1e-12, atol=1e-12)


def test_every_token_its_own_sequence():
    B, L, H, P, G, N = 1, 9, 2, 3, 1, 4
    d = _inputs(9, B, L, H, P, G, N)
    seq = np.arange(L, dtype=np.int32)[None]
    y, f = recurrence_varlen(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], seq)
    for t in range(1, L):
        for h in range(H):
            cb = float(d["Cm"][0, t, 0] @ d["Bm"][0, t, 0])
            np.testing.assert_allclose(y[0, t, h], (d["dt"][0, t, h] * cb + d["D"][h]) * d["x"][0, t, h],
                                       rtol=1e-12, atol=1e-12)
    # the final state is the last token's input term alone
    for h in range(H):
        want = d["dt"][0, L - 1, h] * np.outer(d["x"][0, L - 1, h], d["Bm"][0, L - 1, 0])
        np.testing.assert_allclose(f[0, h], want, rtol=1e-12, atol=1e-12)


def test_sequences_do_not_leak():
    B, L, H, P, G, N = 1, 24, 2, 3, 1, 4
    d = _inputs(10, B, L, H, P, G, N)
    seq = si.make_seq_idx(B, L, lengths=[[8, 9, 7]])
    y, f = recurrence_varlen(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["D"], d["init"], seq)
    moved = {k: (None if v is None else v.copy()) for k, v in d.items()}
    for k in ("x", "Bm", "Cm"):
        moved[k][0, 8:17] += 1.0
    moved["dt"][0, 8:17] *= 2.0
    y2, f2 = recurrence_varlen(moved["x"], moved["dt"], moved["A"], moved["Bm"], moved["Cm"], moved["D"],
                               moved["init"], seq)
    assert np.array_equal(y[0, :8], y2[0, :8]) and np.array_equal(y[0, 17:], y2[0, 17:])
    assert np.array_equal(f, f2)
    assert not np.allclose(y[0, 8:17], y2[0, 8:17])


def test_generator_rows():
    seq = si.make_seq_idx(3, 5000, mean_len=300.0, seed=4)
    assert seq.dtype == np.int32 and seq.shape == (3, 5000)
    for b in range(3):
        assert seq[b, 0] == 0 and np.all(np.diff(seq[b]) >= 0) and np.all(np.diff(seq[b]) <= 1)
        runs = run_bounds(seq[b])
        assert sum(e - s for s, e in runs) == 5000 and len(runs) > 3
    fixed = si.make_seq_idx(1, 10, lengths=[[4, 2]])
    assert fixed.tolist() == [[0, 0, 0, 0, 1, 1, 2, 2, 2, 2]]
