"""fp64 numpy forms of the SSD scan used to pin the recurrence oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Two forms, each written from its own passage of the pages and sharing no code
with the C recurrence:

* ``quadratic`` -- the materialised sequence-transformation matrix.  The
  "Mamba-2" note (section "writing the SSM as a matrix") unrolls the recurrence
  into y = M x with M_ji = C_j^T A_j ... A_{i+1} B_i (lower triangular, zero
  initial state); with a scalar decay (section "reducing A to a number") this
  is M = L o (C B^T) with L_ji = a_j x ... x a_{i+1} for j >= i, 0 above the
  diagonal.  Here a_k = exp(dt_k A_h) and the input term carries dt_i, so
  M_ji = (Cm_j . Bm_i) * exp(sum_{k=i+1}^{j} dt_k A_h) * dt_i.  The segment
  sums are taken directly over (i, j], never as differences of prefix sums.
  An initial state h_{-1} adds exp(sum_{k=0}^{j} dt_k A_h) * Cm_j^T h_{-1} to
  row j.  Only for tiny L (the matrix is L x L per head).

* ``chunked`` -- the block decomposition of M: the sequence is cut into
  blocks of ``chunk`` tokens (the last may be shorter); the "Mamba-2 model
  walkthrough" (section 6.1, and 6.2 describing the paper's minimal listing)
  computes (1) the diagonal blocks in quadratic form, (2) each block's state
  from its inputs, (3) the state passed from block to block, and (4) each
  block's output contribution from the state that enters it; the two output
  parts are summed.  The same four steps, in the same order, in float64.

Layouts: x [B,L,H,P], dt [B,L,H], A [H], Bm/Cm [B,L,G,N], D [H],
init [B,H,P,N] or None.  Returns (y [B,L,H,P], final [B,H,P,N]).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _segment_sums(a: np.ndarray) -> np.ndarray:
    """seg[j, i] = sum_{k=i+1}^{j} a[k] for j >= i (0 on the diagonal), and
    -inf above the diagonal; each column summed directly from its start."""
    n = a.shape[0]
    seg = np.full((n, n), -np.inf)
    for i in range(n):
        seg[i, i] = 0.0
        if i + 1 < n:
            seg[i + 1:, i] = np.cumsum(a[i + 1:])
    return seg


def decay_mask(dt_col: np.ndarray, A_h: float) -> np.ndarray:
    """The mask L of one head: L[j, i] = exp(sum_{k=i+1}^{j} dt_k A_h), j >= i."""
    return np.exp(_segment_sums(np.asarray(dt_col, dtype=np.float64) * float(A_h)))


def quadratic(x, dt, A, Bm, Cm, D, init: Optional[np.ndarray] = None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Materialised matrix form y = M x + D x (+ initial-state term)."""
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bsz, L, H, P))
    final = np.zeros((Bsz, H, P, N))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            a = dt[b, :, h] * A[h]
            Lm = np.exp(_segment_sums(a))                     # [L, L]
            CB = Cm[b, :, g, :] @ Bm[b, :, g, :].T            # [L, L]
            M = Lm * CB * dt[b, :, h][None, :]
            y[b, :, h, :] = M @ x[b, :, h, :] + D[h] * x[b, :, h, :]
            # final state: the last row of the state-valued transform
            last = Lm[L - 1, :] * dt[b, :, h] if L > 0 else np.zeros(0)
            final[b, h] = (x[b, :, h, :] * last[:, None]).T @ Bm[b, :, g, :]
            if init is not None:
                head = np.exp(np.cumsum(a))                   # sum_{k=0}^{j} a_k
                y[b, :, h, :] += head[:, None] * (Cm[b, :, g, :] @ init[b, h].T)
                if L > 0:
                    final[b, h] += head[-1] * init[b, h]
                else:
                    final[b, h] += init[b, h]
    return y, final


def chunked(x, dt, A, Bm, Cm, D, init: Optional[np.ndarray] = None, chunk: int = 64
            ) -> Tuple[np.ndarray, np.ndarray]:
    """Block decomposition in four steps (diagonal blocks, block states,
    block-to-block state passing, state-to-output), in float64."""
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bsz, L, H, P))
    final = np.zeros((Bsz, H, P, N))
    starts = list(range(0, L, chunk))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            a_all = dt[b, :, h] * A[h]
            # step 1: diagonal blocks, quadratic (attention-like) form
            y_diag = np.zeros((L, P))
            for s in starts:
                e = min(s + chunk, L)
                seg = _segment_sums(a_all[s:e])
                G_blk = Cm[b, s:e, g, :] @ Bm[b, s:e, g, :].T
                Mblk = np.exp(seg) * G_blk * dt[b, s:e, h][None, :]
                y_diag[s:e] = Mblk @ x[b, s:e, h, :]
            # step 2: the state each block produces from its own inputs
            states = []
            decays = []
            for s in starts:
                e = min(s + chunk, L)
                q = e - s
                a = a_all[s:e]
                # decay from token i to the end of the block: sum_{k=i+1}^{e-1} a_k
                to_end = np.array([np.sum(a[i + 1:q]) for i in range(q)])
                w = np.exp(to_end) * dt[b, s:e, h]
                states.append((x[b, s:e, h, :] * w[:, None]).T @ Bm[b, s:e, g, :])
                decays.append(np.exp(np.sum(a)))
            # step 3: pass the state from block to block
            H_in = []
            cur = np.zeros((P, N)) if init is None else init[b, h].astype(np.float64).copy()
            for c in range(len(starts)):
                H_in.append(cur)
                cur = decays[c] * cur + states[c]
            final[b, h] = cur
            # step 4: the output of each block from the state entering it
            y_off = np.zeros((L, P))
            for c, s in enumerate(starts):
                e = min(s + chunk, L)
                a = a_all[s:e]
                from_start = np.array([np.sum(a[:i + 1]) for i in range(e - s)])
                y_off[s:e] = np.exp(from_start)[:, None] * (Cm[b, s:e, g, :] @ H_in[c].T)
            y[b, :, h, :] = y_diag + y_off + D[h] * x[b, :, h, :]
    return y, final
