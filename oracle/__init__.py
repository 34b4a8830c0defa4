"""fp64 CPU oracle for the Mamba-2 SSD scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library ``libssd`` and never imports it.

Forms:

* ``recurrence`` -- the token-by-token recurrence in C (``ssd_oracle.c``,
  OpenMP over (batch, head)); the primary oracle.
* ``step`` -- one decode token, the same update applied once, in C.
* ``quadratic`` / ``chunked`` -- numpy fp64 matrix and block-decomposition
  forms (``forms.py``), used to pin the recurrence.
* ``recurrence_bwd`` -- gradients of the scan: the adjoint of the recurrence,
  run backwards in time (``backward.py``, numpy), pinned by finite
  differences of ``recurrence``, exact adjointness and closed forms.
* ``recurrence_varlen`` -- packed rows of independent sequences (``seq_idx``),
  each run of equal values scanned on its own (``varlen.py``).
* ``block_prologue`` / ``gated_norm`` -- the steps before and after the scan
  in a Mamba-2 block (``block.py``).
* ``selective_scan`` -- the Mamba-1 selective scan with diagonal A (``s6.py``).

Every function takes float64 arrays (the values the GPU receives, widened
exactly) and returns float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

from .forms import chunked, decay_mask, quadratic  # noqa: F401
from .backward import recurrence_bwd  # noqa: F401
from .varlen import recurrence_varlen, run_bounds  # noqa: F401
from .block import block_prologue, gated_norm  # noqa: F401
from .s6 import selective_scan  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "libssd_oracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle with gcc (always recompiles)."""
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_ssd_recurrence.argtypes = [i64] * 6 + [dp] * 9 + [ip, i64]
    lib.oracle_ssd_recurrence.restype = ctypes.c_int
    lib.oracle_ssd_step.argtypes = [i64] * 5 + [dp] * 8 + [ip, i64]
    lib.oracle_ssd_step.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_load().oracle_num_threads())


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _bh_list(bh: Optional[Sequence[int]]):
    if bh is None:
        return None, None, 0
    arr = np.ascontiguousarray(np.asarray(bh, dtype=np.int64))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(arr.size)


def recurrence(x, dt, A, Bm, Cm, D, init=None, bh: Optional[Sequence[int]] = None
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token recurrence.  Shapes: x [B,L,H,P], dt [B,L,H], A [H],
    Bm/Cm [B,L,G,N], D [H], init [B,H,P,N] or None.  With ``bh`` (a list of
    b*H+h indices) only those (batch, head) pairs are computed; the others are
    returned as NaN.  Returns (y [B,L,H,P], final [B,H,P,N])."""
    x, dt, A, Bm, Cm, D, init = map(_f64, (x, dt, A, Bm, Cm, D, init))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    assert dt.shape == (Bsz, L, H) and A.shape == (H,) and D.shape == (H,)
    assert Bm.shape == (Bsz, L, G, N) and Cm.shape == Bm.shape
    assert init is None or init.shape == (Bsz, H, P, N)
    y = np.full((Bsz, L, H, P), np.nan)
    final = np.full((Bsz, H, P, N), np.nan)
    keep, bh_p, n_bh = _bh_list(bh)
    rc = _load().oracle_ssd_recurrence(Bsz, L, H, P, G, N, _dptr(x), _dptr(dt), _dptr(A),
                                       _dptr(Bm), _dptr(Cm), _dptr(D), _dptr(init),
                                       _dptr(y), _dptr(final), bh_p, n_bh)
    del keep
    if rc != 0:
        raise ValueError("oracle_ssd_recurrence rejected its arguments")
    return y, final


def step(state, x, dt, A, Bm, Cm, D, bh: Optional[Sequence[int]] = None) -> np.ndarray:
    """One decode token.  ``state`` [B,H,P,N] float64 is updated in place;
    x [B,H,P], dt [B,H], Bm/Cm [B,G,N].  Returns y [B,H,P] (NaN for pairs not
    in ``bh``)."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags.c_contiguous):
        raise TypeError("state must be a C-contiguous float64 array (updated in place)")
    x, dt, A, Bm, Cm, D = map(_f64, (x, dt, A, Bm, Cm, D))
    Bsz, H, P, N = state.shape
    G = Bm.shape[1]
    assert x.shape == (Bsz, H, P) and dt.shape == (Bsz, H) and Bm.shape == (Bsz, G, N)
    y = np.full((Bsz, H, P), np.nan)
    keep, bh_p, n_bh = _bh_list(bh)
    rc = _load().oracle_ssd_step(Bsz, H, P, G, N, _dptr(state), _dptr(x), _dptr(dt), _dptr(A),
                                 _dptr(Bm), _dptr(Cm), _dptr(D), _dptr(y), bh_p, n_bh)
    del keep
    if rc != 0:
        raise ValueError("oracle_ssd_step rejected its arguments")
    return y
