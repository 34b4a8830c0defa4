"""Helpers for the GPU parity tests: seeded inputs onto the device, the oracle
on the same values, and the error metric.

Error metric: per output tensor, max |got - ref| / max |ref| (the oracle's
max magnitude), with ref the float64 oracle on exactly the values the GPU
received.  Limits: 2e-2 when x, Bm, Cm, y are bfloat16 (products inside a
block use bfloat16 operands, accumulation is float32); 1e-4 in float32 mode.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import ssd_inputs as si  # noqa: E402

TOL = {"bf16": 2e-2, "fp32": 1e-4}
TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / scale)


def to_device(d, dtype: str, device="cuda"):
    """Stored float32 values -> device tensors (x, Bm, Cm in the run's dtype)."""
    td = TORCH_DTYPE[dtype]
    out = {}
    for k, v in d.items():
        if v is None:
            out[k] = None
        elif k in ("x", "Bm", "Cm"):
            out[k] = torch.from_numpy(v).to(device=device, dtype=td)
        else:
            out[k] = torch.from_numpy(v).to(device=device, dtype=torch.float32)
    return out


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_scan(d, bh=None):
    f = si.as_f64(d)
    return oracle.recurrence(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], bh=bh)


def gpu_scan(dd, chunk, algo="auto", **kw):
    import selective_state_space_chunk_amd as ssd
    y, fin = ssd.ssd_chunk_scan_fwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"],
                                    dd["init"], chunk, algo=algo, **kw)
    torch.cuda.synchronize()
    return y, fin


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
