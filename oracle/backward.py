"""fp64 gradients of the SSD scan: the adjoint (reverse-mode derivative) of
the token recurrence, written out as its own backwards loop.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library and does not call the forward oracle.

The recurrence is the one the "Mamba-2" note unrolls (section "writing the
SSM as a matrix"), with one decay per head (section "reducing A to a
number") and the input term carrying dt:

    S_t = a_t S_{t-1} + dt_t x_t (outer) Bm_t,   a_t = exp(dt_t A_h),   S_{-1} = init
    y_t = S_t Cm_t + D_h x_t

For the scalar  <dy, y> + <dfinal, S_{L-1}>  every gradient follows from one
pass backwards in time over the adjoint G_t = d/dS_t:

    G_{L-1} = dfinal + dy_{L-1} (outer) Cm_{L-1}
    G_t     = a_{t+1} G_{t+1} + dy_t (outer) Cm_t
    dCm_t  += S_t^T dy_t                           (summed over the heads of the group)
    dx_t    = dt_t G_t Bm_t + D_h dy_t
    dBm_t  += dt_t G_t^T x_t                       (summed over the heads of the group)
    ddt_t   = <G_t, x_t (outer) Bm_t> + A_h a_t <G_t, S_{t-1}>
    dA_h   += dt_t a_t <G_t, S_{t-1}>
    dD_h   += <dy_t, x_t>
    dinit   = a_0 G_0

Layouts as the forward: x, dy [B,L,H,P]; dt [B,L,H]; A, D [H]; Bm, Cm
[B,L,G,N]; init, dfinal [B,H,P,N] or None.  Head h uses group h // (H/G).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def recurrence_bwd(x, dt, A, Bm, Cm, D, init: Optional[np.ndarray], dy,
                   dfinal: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of <dy, y> + <dfinal, final> with respect to every input.
    Returns a dict with dx, ddt, dA, dBm, dCm, dD, dinit (all float64)."""
    x, dt, A, Bm, Cm, D, dy = (np.asarray(v, dtype=np.float64) for v in (x, dt, A, Bm, Cm, D, dy))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    out = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dA": np.zeros(H),
           "dBm": np.zeros_like(Bm), "dCm": np.zeros_like(Cm), "dD": np.zeros(H),
           "dinit": np.zeros((Bsz, H, P, N))}
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            a = np.exp(dt[b, :, h] * A[h])
            # forward states S_{-1} .. S_{L-1}
            S = np.zeros((L + 1, P, N))
            if init is not None:
                S[0] = np.asarray(init[b, h], dtype=np.float64)
            for t in range(L):
                S[t + 1] = a[t] * S[t] + dt[b, t, h] * np.outer(x[b, t, h], Bm[b, t, g])
            Gt = np.zeros((P, N)) if dfinal is None else np.array(dfinal[b, h], dtype=np.float64)
            for t in range(L - 1, -1, -1):
                Gt = Gt + np.outer(dy[b, t, h], Cm[b, t, g])          # G_t
                out["dCm"][b, t, g] += S[t + 1].T @ dy[b, t, h]
                out["dx"][b, t, h] = dt[b, t, h] * (Gt @ Bm[b, t, g]) + D[h] * dy[b, t, h]
                out["dBm"][b, t, g] += dt[b, t, h] * (Gt.T @ x[b, t, h])
                gs = float(np.sum(Gt * S[t]))                          # <G_t, S_{t-1}>
                out["ddt"][b, t, h] = float(x[b, t, h] @ Gt @ Bm[b, t, g]) + A[h] * a[t] * gs
                out["dA"][h] += dt[b, t, h] * a[t] * gs
                out["dD"][h] += float(dy[b, t, h] @ x[b, t, h])
                Gt = a[t] * Gt                                         # d/dS_{t-1}
            out["dinit"][b, h] = Gt
    return out
