"""Seeded synthetic inputs for the SSD scan, shared by the oracle tests, the GPU
parity tests and the benchmark.

This module only draws random numbers and rounds them to the storage precision
of a run.  It holds none of the scan's arithmetic, so that the CPU oracle and
the HIP path, which share nothing else, can be fed exactly the same values.

Workload shapes are Mamba-2 layer shapes (the "Mamba-2" note, section on the
Mamba-2 block: head dim P = 64, B and C shared by the heads of a group; the
130M and 2.7B layers use d_model 768 and 2560 with expand 2).  Value
distributions, per tensor:

* x ~ N(0, 1)                         [B, L, H, P]
* Bm, Cm ~ N(0, 1) / sqrt(N)          [B, L, G, N]
* dt = softplus(N(0, 1) - 4)          [B, L, H]  (median ~0.018; the step size
  of the selection mechanism is a softplus of a projection, "Mamba" reading
  notes section 3.2; here the projection is replaced by a Gaussian)
* A_h = -exp(U(log 1, log 16))        [H]  (negative scalar per head)
* D ~ N(0, 1)                         [H]
* init_state ~ N(0, 0.1^2)            [B, H, P, N]  (when the workload asks)

Each tensor is drawn from ``numpy.random.default_rng([seed, tensor_id])`` in
float64 and then rounded to its storage type: x, Bm, Cm to bfloat16 (round to
nearest even) in bf16 runs, to float32 in fp32 runs; dt, A, D and the states to
float32 always.  The rounded values, widened back to float64, are what the
oracle sees; the same rounded values go to the GPU.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

# tensor ids for default_rng([seed, id]); fixed so that every consumer draws the
# same stream for the same tensor
_TID = {"x": 1, "dt": 2, "A": 3, "Bm": 4, "Cm": 5, "D": 6, "init": 7,
        "step_x": 11, "step_dt": 12, "step_Bm": 14, "step_Cm": 15,
        "dy": 21, "dfinal": 22, "seq": 23, "zxbcdt": 24, "conv_w": 25, "conv_b": 26, "dt_bias": 27, "norm_w": 28, "norm_b": 29, "ynorm": 30, "s6x": 31, "s6dt": 32, "s6A": 33, "s6B": 34, "s6C": 35, "s6D": 36, "s6init": 37}

SEED_BASE = 20240531


@dataclasses.dataclass(frozen=True)
class Workload:
    """One seeded workload: the shape, the storage dtype and the init rule."""
    name: str
    B: int
    L: int
    H: int
    P: int
    N: int
    G: int
    chunk: int
    dtype: str            # "bf16" or "fp32": storage type of x, Bm, Cm, y
    init: bool            # draw a nonzero initial state
    steps: int = 0        # decode workloads: number of consecutive tokens
    index: int = 0        # seed offset

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def tokens(self) -> int:
        return self.B * self.L


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 scan
    "tiny_fp32": Workload("tiny_fp32", B=1, L=256, H=4, P=16, N=16, G=1, chunk=64,
                          dtype="fp32", init=False, index=0),
    # Mamba-2 130M layer: d_model 768, expand 2 -> 24 heads x 64
    "m2_130m": Workload("m2_130m", B=8, L=2048, H=24, P=64, N=128, G=1, chunk=256,
                        dtype="bf16", init=False, index=1),
    # Mamba-2 2.7B layer: d_model 2560, expand 2 -> 80 heads x 64, random init state
    "m2_2p7b": Workload("m2_2p7b", B=4, L=4096, H=80, P=64, N=128, G=1, chunk=256,
                        dtype="bf16", init=True, index=2),
    # long sequence, 130M layer shape
    "long_n128": Workload("long_n128", B=1, L=65536, H=24, P=64, N=128, G=1, chunk=256,
                          dtype="bf16", init=False, index=3),
    "long_n256": Workload("long_n256", B=1, L=65536, H=24, P=64, N=256, G=1, chunk=256,
                          dtype="bf16", init=False, index=3),
    # the 2.7B layer's 5120 inner channels as 40 heads of the other head dim
    # the pages give (P = 128)
    "m2_2p7b_p128": Workload("m2_2p7b_p128", B=4, L=4096, H=40, P=128, N=128, G=1, chunk=256,
                             dtype="bf16", init=True, index=5),
    # recurrent decode: 1024 consecutive single-token steps from a random state
    "decode_2p7b": Workload("decode_2p7b", B=256, L=1, H=80, P=64, N=128, G=1, chunk=256,
                            dtype="bf16", init=True, steps=1024, index=4),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 holding
    exactly representable bfloat16 values.  NaN/Inf are not expected here."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([seed, _TID[name]])


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z) written to stay finite for large |z|
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type; returns float32."""
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "fp32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_scan_inputs(B: int, L: int, H: int, P: int, N: int, G: int = 1, *,
                     dtype: str = "bf16", init: bool = False, seed: int = SEED_BASE,
                     regime: str = "default") -> Dict[str, Optional[np.ndarray]]:
    """Seeded chunk-scan inputs, each a float32 array holding the stored values.

    ``regime`` selects the dt/A distribution:

    * ``"default"``: the workload distributions listed in the module docstring.
    * ``"long_memory"``: dt ~ U(0.3, 1.5), A_h = -U(0.05, 0.5) -- slow decay,
      so errors in the state passed between chunks are not hidden by forgetting.
    * ``"no_decay"``: A = 0 -- states are passed at full magnitude.
    * ``"decay_bursts"``: the default distributions, with dt multiplied by 40
      inside random 96-token stretches (about a quarter of every row and head):
      stretches where the state is all but erased within a few tokens, next
      to ordinary ones.
    * ``"strong_decay"``: dt ~ U(0.3, 1.5), A_h = -U(1, 16) -- every step
      forgets most of the state.
    """
    if H % G:
        raise ValueError("H must be a multiple of G")
    out: Dict[str, Optional[np.ndarray]] = {}
    out["x"] = _store(_rng(seed, "x").standard_normal((B, L, H, P)), dtype)
    s = 1.0 / math.sqrt(N)
    out["Bm"] = _store(_rng(seed, "Bm").standard_normal((B, L, G, N)) * s, dtype)
    out["Cm"] = _store(_rng(seed, "Cm").standard_normal((B, L, G, N)) * s, dtype)
    if regime == "default":
        dt = _softplus(_rng(seed, "dt").standard_normal((B, L, H)) - 4.0)
        A = -np.exp(_rng(seed, "A").uniform(math.log(1.0), math.log(16.0), H))
    elif regime == "long_memory":
        dt = _rng(seed, "dt").uniform(0.3, 1.5, (B, L, H))
        A = -_rng(seed, "A").uniform(0.05, 0.5, H)
    elif regime == "no_decay":
        dt = _softplus(_rng(seed, "dt").standard_normal((B, L, H)) - 4.0)
        A = np.zeros(H)
    elif regime == "decay_bursts":
        r = _rng(seed, "dt")
        dt = _softplus(r.standard_normal((B, L, H)) - 4.0)
        A = -np.exp(_rng(seed, "A").uniform(math.log(1.0), math.log(16.0), H))
        nb = max(1, L // 384)
        for b in range(B):
            for h in range(H):
                for s0 in r.integers(0, max(1, L), nb):
                    dt[b, s0:s0 + 96, h] *= 40.0
    elif regime == "strong_decay":
        dt = _rng(seed, "dt").uniform(0.3, 1.5, (B, L, H))
        A = -_rng(seed, "A").uniform(1.0, 16.0, H)
    else:
        raise ValueError(f"unknown regime {regime!r}")
    out["dt"] = np.ascontiguousarray(dt, dtype=np.float32)
    out["A"] = np.ascontiguousarray(A, dtype=np.float32)
    out["D"] = np.ascontiguousarray(_rng(seed, "D").standard_normal(H), dtype=np.float32)
    if init:
        out["init"] = np.ascontiguousarray(
            _rng(seed, "init").standard_normal((B, H, P, N)) * 0.1, dtype=np.float32)
    else:
        out["init"] = None
    return out


def make_step_inputs(B: int, H: int, P: int, N: int, G: int = 1, *, step: int = 0,
                     dtype: str = "bf16", seed: int = SEED_BASE) -> Dict[str, np.ndarray]:
    """Seeded inputs of decode token number ``step`` (one token per call).

    Returns x [B, H, P], dt [B, H], Bm/Cm [B, G, N], A [H] and D [H], with the
    same distributions and rounding as the scan inputs.  Each step draws from
    its own stream, so a long run of steps never has to be held in memory."""
    def rng(name):
        return np.random.default_rng([seed, _TID[name], step])
    out: Dict[str, np.ndarray] = {}
    out["x"] = _store(rng("step_x").standard_normal((B, H, P)), dtype)
    s = 1.0 / math.sqrt(N)
    out["Bm"] = _store(rng("step_Bm").standard_normal((B, G, N)) * s, dtype)
    out["Cm"] = _store(rng("step_Cm").standard_normal((B, G, N)) * s, dtype)
    out["dt"] = np.ascontiguousarray(
        _softplus(rng("step_dt").standard_normal((B, H)) - 4.0), dtype=np.float32)
    out["A"] = np.ascontiguousarray(
        -np.exp(_rng(seed, "A").uniform(math.log(1.0), math.log(16.0), H)), dtype=np.float32)
    out["D"] = np.ascontiguousarray(_rng(seed, "D").standard_normal(H), dtype=np.float32)
    return out


def make_step_state(B: int, H: int, P: int, N: int, *, seed: int = SEED_BASE) -> np.ndarray:
    """Starting decode state [B, H, P, N] ~ N(0, 0.1^2), float32."""
    return np.ascontiguousarray(
        _rng(seed, "init").standard_normal((B, H, P, N)) * 0.1, dtype=np.float32)


def workload_scan_inputs(w: Workload, regime: str = "default"):
    return make_scan_inputs(w.B, w.L, w.H, w.P, w.N, w.G, dtype=w.dtype, init=w.init,
                            seed=w.seed, regime=regime)


def make_grad_inputs(B: int, L: int, H: int, P: int, N: int, *, dtype: str = "bf16",
                     dfinal: bool = True, seed: int = SEED_BASE) -> Dict[str, Optional[np.ndarray]]:
    """Seeded upstream gradients for the backward scan: dy ~ N(0,1) in the
    storage dtype of y [B,L,H,P], and dfinal ~ N(0, 0.1) float32 [B,H,P,N]
    (or None)."""
    out: Dict[str, Optional[np.ndarray]] = {}
    out["dy"] = _store(_rng(seed, "dy").standard_normal((B, L, H, P)), dtype)
    out["dfinal"] = (np.ascontiguousarray(_rng(seed, "dfinal").standard_normal((B, H, P, N)) * 0.1,
                                          dtype=np.float32) if dfinal else None)
    return out


def make_seq_idx(B: int, L: int, *, mean_len: float = 512.0, seed: int = SEED_BASE,
                 lengths: Optional[Sequence[Sequence[int]]] = None) -> np.ndarray:
    """Sequence index of every token of packed rows, int32 [B, L]: row b holds
    documents 0, 1, 2, ... one after another.  With ``lengths`` the documents
    of row b have those lengths (the last one cut or extended to fill L);
    otherwise lengths are drawn log-normally with median ``mean_len`` (spread
    of a factor e), at least 1 token, the last document cut at the row's end."""
    out = np.zeros((B, L), dtype=np.int32)
    rng = _rng(seed, "seq")
    for b in range(B):
        t, k = 0, 0
        row_lengths = list(lengths[b]) if lengths is not None else None
        while t < L:
            if row_lengths is not None:
                n = row_lengths[k] if k < len(row_lengths) else L - t
            else:
                n = int(max(1, round(float(rng.lognormal(np.log(mean_len), 1.0)))))
            n = max(1, min(n, L - t))
            out[b, t:t + n] = k
            t += n
            k += 1
    return out


def make_block_inputs(B: int, L: int, H: int, P: int, G: int, N: int, W: int = 4, *,
                      seed: int = SEED_BASE) -> Dict[str, np.ndarray]:
    """Seeded inputs of the steps around the scan in a Mamba-2 block: the
    projection output zxbcdt [B, L, 2HP + 2GN + H] ~ N(0, 1) in bfloat16,
    conv taps [HP + 2GN, W] ~ N(0, 1/W) and bias ~ N(0, 0.1) (fp32), dt_bias
    [H] so that softplus(dt_raw + dt_bias) spans small and large steps, norm
    weight ~ 1 + N(0, 0.1) and bias ~ N(0, 0.1) over the HP channels, and a
    scan output y [B, L, H, P] ~ N(0, 1) in bfloat16."""
    HP, GN = H * P, G * N
    C = HP + 2 * GN
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {
        "zxbcdt": round_bf16(_rng(seed, "zxbcdt").standard_normal((B, L, 2 * HP + 2 * GN + H))),
        "conv_w": f32(_rng(seed, "conv_w").standard_normal((C, W)) / np.sqrt(W)),
        "conv_b": f32(_rng(seed, "conv_b").standard_normal(C) * 0.1),
        "dt_bias": f32(_rng(seed, "dt_bias").uniform(-4.0, 1.0, H)),
        "norm_w": f32(1.0 + 0.1 * _rng(seed, "norm_w").standard_normal(HP)),
        "norm_b": f32(0.1 * _rng(seed, "norm_b").standard_normal(HP)),
        "y": round_bf16(_rng(seed, "ynorm").standard_normal((B, L, H, P))),
    }


def make_s6_inputs(B: int, L: int, Dch: int, N: int, G: int = 1, *, init: bool = True,
                   seed: int = SEED_BASE) -> Dict[str, Optional[np.ndarray]]:
    """Seeded inputs of the Mamba-1 selective scan: x ~ N(0, 1) and dt =
    softplus(N(-1, 1)) in bfloat16 [B, L, Dch]; A = -exp(U(-1, 1.5)) fp32
    [Dch, N] (decays from mild to strong); Bm, Cm ~ N(0, 1) bfloat16
    [B, L, G, N]; D ~ N(0, 1) fp32 [Dch]; init ~ N(0, 0.3) fp32 [B, Dch, N]."""
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return {
        "x": round_bf16(_rng(seed, "s6x").standard_normal((B, L, Dch))),
        "dt": round_bf16(_softplus(_rng(seed, "s6dt").standard_normal((B, L, Dch)) - 1.0)),
        "A": f32(-np.exp(_rng(seed, "s6A").uniform(-1.0, 1.5, (Dch, N)))),
        "Bm": round_bf16(_rng(seed, "s6B").standard_normal((B, L, G, N))),
        "Cm": round_bf16(_rng(seed, "s6C").standard_normal((B, L, G, N))),
        "D": f32(_rng(seed, "s6D").standard_normal(Dch)),
        "init": f32(_rng(seed, "s6init").standard_normal((B, Dch, N)) * 0.3) if init else None,
    }


def as_f64(arrs: Dict[str, Optional[np.ndarray]]) -> Dict[str, Optional[np.ndarray]]:
    """Widen stored values to float64 for the oracle (exact)."""
    return {k: (None if v is None else np.ascontiguousarray(v, dtype=np.float64))
            for k, v in arrs.items()}
