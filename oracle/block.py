"""fp64 oracle for the steps on either side of the scan in a Mamba-2 block.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with
the HIP library.

The "Mamba-2" note (section "Mamba-2 block") describes the parallel block:
one projection yields the gate input z, X, B, C and the step dt at once; the
scan's output is multiplied by the gate and normalised before the output
projection.  The "Mamba-2" walkthrough (section 7.2) names the normalisation
a GroupNorm, chosen so that tensor-parallel ranks need not communicate.
Readings taken (the pages fix no more):

* the projection output of one token is laid out [z (H P) | x (H P) |
  Bm (G N) | Cm (G N) | dt (H)];
* x, Bm and Cm pass through a causal depthwise convolution of width W (zero
  before the first token, a bias per channel) and SiLU, as the Mamba block
  makes X by a convolution and an activation ("Mamba" note, figure of the two
  blocks);
* dt = softplus(dt_raw + dt_bias);
* the gate is SiLU(z); the norm works on each of ``ngroups`` equal groups of
  the H P channels of one token: mean-centred with variance (GroupNorm) or,
  with ``center=False``, root-mean-square only; then a per-channel weight and
  an optional bias.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def silu(v: np.ndarray) -> np.ndarray:
    return v / (1.0 + np.exp(-v))


def softplus(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def block_prologue(zxbcdt, conv_w, conv_b, dt_bias, H: int, P: int, G: int, N: int) -> Dict[str, np.ndarray]:
    """zxbcdt [B, L, 2HP + 2GN + H]; conv_w [C, W] over the C = HP + 2GN channels;
    conv_b [C]; dt_bias [H].  Returns z [B,L,HP], x [B,L,H,P], Bm, Cm
    [B,L,G,N] and dt [B,L,H]."""
    v = np.asarray(zxbcdt, dtype=np.float64)
    w = np.asarray(conv_w, dtype=np.float64)
    cb = np.asarray(conv_b, dtype=np.float64)
    Bsz, L, _ = v.shape
    d, gn = H * P, G * N
    C = d + 2 * gn
    W = w.shape[1]
    assert v.shape[2] == 2 * d + 2 * gn + H and w.shape == (C, W) and cb.shape == (C,)
    z = v[:, :, :d]
    xbc = v[:, :, d:d + C]
    dt_raw = v[:, :, d + C:]
    conv = np.broadcast_to(cb, (Bsz, L, C)).copy()
    for k in range(W):
        lag = W - 1 - k              # tap k multiplies the input lag tokens back
        if lag == 0:
            conv += w[:, k] * xbc
        elif lag < L:
            conv[:, lag:] += w[:, k] * xbc[:, :L - lag]
    act = silu(conv)
    return {"z": z.copy(),
            "x": act[:, :, :d].reshape(Bsz, L, H, P),
            "Bm": act[:, :, d:d + gn].reshape(Bsz, L, G, N),
            "Cm": act[:, :, d + gn:].reshape(Bsz, L, G, N),
            "dt": softplus(dt_raw + np.asarray(dt_bias, dtype=np.float64))}


def gated_norm(y, z, weight, bias: Optional[np.ndarray], ngroups: int, eps: float, center: bool) -> np.ndarray:
    """y, z [T, D]; weight (and bias) [D].  Returns the normalised gated
    output [T, D]."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    T, D = y.shape
    assert D % ngroups == 0
    g = (y * silu(z)).reshape(T, ngroups, D // ngroups)
    if center:
        g = g - g.mean(axis=2, keepdims=True)
    g = g / np.sqrt(np.mean(g * g, axis=2, keepdims=True) + eps)
    out = g.reshape(T, D) * np.asarray(weight, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)
    return out
