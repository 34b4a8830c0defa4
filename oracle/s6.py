"""fp64 oracle for the Mamba-1 selective scan (S6): one decay per channel and
state, diagonal A.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library.

The "Mamba" reading notes give the recurrence h_t = Abar h_{t-1} + Bbar x_t,
y_t = C h_t (section 2.2, with the zero-order-hold rule Abar = exp(dt A),
Bbar = (dt A)^-1 (exp(dt A) - I) dt B), and make dt, B and C functions of
the input token (section 3.2, selection).  With a diagonal A every channel d
and state n is a scalar recurrence:

    a = exp(dt_t[d] A[d, n])
    h_t[d, n] = a h_{t-1}[d, n] + bbar x_t[d]
    y_t[d] = sum_n Cm_t[n] h_t[d, n] + D[d] x_t[d]

with bbar = (a - 1) / A[d, n] * Bm_t[n] (zero-order hold; its limit dt Bm_t[n]
where A = 0) or, with ``zoh=False``, bbar = dt_t[d] Bm_t[n] (the simpler
form the SSD scan uses).  Channel d reads group d // (Dch / G) of Bm and Cm.
Shapes: x, dt [B, L, Dch]; A [Dch, N]; Bm, Cm [B, L, G, N]; D [Dch] or None;
init [B, Dch, N] or None.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def selective_scan(x, dt, A, Bm, Cm, D: Optional[np.ndarray], init: Optional[np.ndarray] = None,
                   zoh: bool = True, channels=None) -> Tuple[np.ndarray, np.ndarray]:
    """Returns (y [B, L, Dch], final state [B, Dch, N]).  With ``channels``
    (a list of channel indices) only those are computed; the rest are NaN."""
    x, dt, A, Bm, Cm = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, Bm, Cm))
    Bsz, L, Dch = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    ch = np.arange(Dch) if channels is None else np.asarray(channels)
    grp = ch // (Dch // G)
    Ac = A[ch]                                            # [c, N]
    h = np.zeros((Bsz, len(ch), N)) if init is None else np.asarray(init, dtype=np.float64)[:, ch].copy()
    y = np.full((Bsz, L, Dch), np.nan)
    Dv = np.zeros(len(ch)) if D is None else np.asarray(D, dtype=np.float64)[ch]
    for t in range(L):
        d = dt[:, t, ch][:, :, None]                      # [B, c, 1]
        a = np.exp(d * Ac)
        if zoh:
            safe = np.where(Ac == 0.0, 1.0, Ac)
            coef = np.where(Ac == 0.0, d, np.expm1(d * Ac) / safe)
        else:
            coef = np.broadcast_to(d, a.shape)
        h = a * h + coef * Bm[:, t, grp, :] * x[:, t, ch][:, :, None]
        y[:, t, ch] = np.sum(Cm[:, t, grp, :] * h, axis=2) + Dv * x[:, t, ch]
    final = np.full((Bsz, Dch, N), np.nan)
    final[:, ch] = h
    return y, final
