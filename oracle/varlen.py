"""fp64 oracle for packed variable-length sequences with a state reset at
every sequence boundary.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library.

The "Mamba" reading notes (section 3.5, the selection mechanism's abilities)
list boundary resetting: independent sequences concatenated into one row must
not leak information into one another; the "Mamba-2-Hybrid" note (section on
long context) raises the same concern for unrelated documents packed together
in long-context training.  Reading taken: a row of ``seq_idx`` values [B, L]
is cut into maximal runs of equal values; each run is an independent
sequence.  The first run of a row starts from the initial state (or zero),
every later run from zero.  y is the concatenation of the runs' outputs and
the final state of a row is that of its last run.

This module implements exactly that definition: it cuts every row at its
boundaries and runs the token recurrence oracle (``oracle.recurrence``) on
each run on its own.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np


def run_bounds(seq_row: np.ndarray) -> List[Tuple[int, int]]:
    """Half-open [start, end) token ranges of the maximal runs of equal values."""
    seq_row = np.asarray(seq_row)
    L = int(seq_row.shape[0])
    if L == 0:
        return []
    cuts = [0] + [t for t in range(1, L) if seq_row[t] != seq_row[t - 1]] + [L]
    return list(zip(cuts[:-1], cuts[1:]))


def recurrence_varlen(x, dt, A, Bm, Cm, D, init: Optional[np.ndarray], seq_idx,
                      bh: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Outputs of packed rows.  Shapes as ``oracle.recurrence`` plus seq_idx
    [B, L] (integers).  With ``bh`` (b*H+h indices) only those pairs are
    computed; the others are NaN.  Returns (y [B,L,H,P], final [B,H,P,N])."""
    from . import recurrence
    x, dt, A, Bm, Cm, D = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, Bm, Cm, D))
    Bsz, L, H, P = x.shape
    N = Bm.shape[3]
    seq_idx = np.asarray(seq_idx)
    assert seq_idx.shape == (Bsz, L)
    y = np.full((Bsz, L, H, P), np.nan)
    final = np.full((Bsz, H, P, N), np.nan)
    for b in range(Bsz):
        heads = list(range(H)) if bh is None else [k - b * H for k in bh if b * H <= k < (b + 1) * H]
        if not heads:
            continue
        runs = run_bounds(seq_idx[b])
        if not runs:
            if init is not None:
                final[b, heads] = np.asarray(init[b, heads], dtype=np.float64)
            else:
                final[b, heads] = 0.0
            continue
        for k, (s, e) in enumerate(runs):
            i0 = None
            if k == 0 and init is not None:
                i0 = np.asarray(init[b:b + 1], dtype=np.float64)
            yk, fk = recurrence(x[b:b + 1, s:e], dt[b:b + 1, s:e], A, Bm[b:b + 1, s:e], Cm[b:b + 1, s:e],
                                D, i0, bh=heads)
            y[b, s:e][:, heads] = yk[0][:, heads]
            if k == len(runs) - 1:
                final[b, heads] = fk[0, heads]
    return y, final
