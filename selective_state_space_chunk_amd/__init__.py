"""libssd -- the Mamba-2 SSD chunk scan and decode step on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/libssd.h``.  It only
marshals arguments: every step of the scan runs in the HIP kernels of
``libssd.so``.  PyTorch supplies device memory and the current stream.  There
is no fallback: if the library is not built, importing the binding's entry
points raises.

Entry points (same names as the C ABI):

* ``ssd_chunk_scan_fwd(x, dt, A, Bm, Cm, D, init_state=None, chunk_size=256)``
  -> ``(y, final_state)``
* ``ssd_chunk_scan_fwd_varlen(x, dt, A, Bm, Cm, D, seq_idx, init_state=None, chunk_size=256)``
  -> ``(y, final_state)``: packed rows, the state reset wherever seq_idx changes
* ``ssd_chunk_scan_bwd(x, dt, A, Bm, Cm, D, init_state, dy, dfinal=None, chunk_size=256)``
  -> dict of gradients dx, ddt, dA, dBm, dCm, dD, dinit
* ``ssd_step(state, x, dt, A, Bm, Cm, D)`` -> ``y`` (``state`` updated in place)
* ``ssd_chunk_scan_workspace_size(B, L, H, P, G, N, chunk_size, dtype)`` and the
  ``_varlen_`` and ``_bwd_`` variants
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libssd.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP, SSD_ERR_TOO_LARGE = range(6)
SSD_DTYPE_F32, SSD_DTYPE_BF16 = 0, 1
# bytes of the static per-device scratch of ssd_chunk_scan_fwd_noalloc (SSD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
ALGOS = {"auto": 0, "reference": 1, "staged": 2, "pipe": 3}

_lib = None


class SSDError(RuntimeError):
    """A libssd call returned a status other than SSD_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libssd.so (built in-tree by ``build.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libssd.so not found at {LIB_PATH}; build it first with "
            "`python -m selective_state_space_chunk_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_char_p
    lib.ssd_chunk_scan_workspace_size.argtypes = [i64] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_workspace_size.restype = sz
    lib.ssd_chunk_scan_workspace_size_algo.argtypes = [i64] * 7 + [ctypes.c_int, ctypes.c_int]
    lib.ssd_chunk_scan_workspace_size_algo.restype = sz
    scan_args = [vp] * 10 + [sz] + [i64] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_fwd.argtypes = scan_args + [vp]
    lib.ssd_chunk_scan_fwd.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_algo.argtypes = scan_args + [ctypes.c_int, vp]
    lib.ssd_chunk_scan_fwd_algo.restype = ctypes.c_int
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [vp] * 9 + [i64] * 7 + [ctypes.c_int, vp]
    lib.ssd_chunk_scan_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_step.argtypes = [vp] * 8 + [i64] * 5 + [ctypes.c_int, vp]
    lib.ssd_step.restype = ctypes.c_int
    lib.ssd_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.ssd_stream_copy.restype = ctypes.c_int
    lib.ssd_chunk_scan_varlen_workspace_size.argtypes = [i64] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_varlen_workspace_size.restype = sz
    lib.ssd_chunk_scan_fwd_varlen.argtypes = [vp] * 11 + [sz] + [i64] * 7 + [ctypes.c_int, vp]
    lib.ssd_chunk_scan_fwd_varlen.restype = ctypes.c_int
    lib.ssd_block_prologue.argtypes = [vp] * 8 + [i64] * 7 + [ctypes.c_int, vp]
    lib.ssd_block_prologue.restype = ctypes.c_int
    lib.ssd_gated_norm.argtypes = [vp, vp, i64, vp, vp, vp, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                   ctypes.c_int, vp]
    lib.ssd_gated_norm.restype = ctypes.c_int
    lib.ssd_selective_scan.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_int, ctypes.c_int, vp]
    lib.ssd_selective_scan.restype = ctypes.c_int
    lib.ssd_chunk_scan_bwd_workspace_size.argtypes = [i64] * 7 + [ctypes.c_int]
    lib.ssd_chunk_scan_bwd_workspace_size.restype = sz
    lib.ssd_chunk_scan_bwd.argtypes = [vp] * 17 + [sz] + [i64] * 7 + [ctypes.c_int, vp]
    lib.ssd_chunk_scan_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().ssd_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != SSD_OK:
        raise SSDError(status, f"{what}: {status_string(status)}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSD_DTYPE_F32
    if t == torch.bfloat16:
        return SSD_DTYPE_BF16
    raise TypeError(f"x, Bm, Cm must be float32 or bfloat16, got {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream_handle(device: torch.device, stream=None):
    return ctypes.c_void_p(_stream(device, stream).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def ssd_chunk_scan_workspace_size(B: int, L: int, H: int, P: int, G: int, N: int,
                                  chunk_size: int, dtype: torch.dtype, algo: str = "auto") -> int:
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}")
    return int(load_library().ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, chunk_size,
                                                                 _dtype_code(dtype), ALGOS[algo]))


_workspaces: Dict[Tuple[int, int], torch.Tensor] = {}


def workspace(nbytes: int, device: torch.device, stream=None) -> torch.Tensor:
    """A device workspace of at least ``nbytes``, cached per (device, stream).

    The library writes its scratch before reading it, so the bytes need no
    initialisation.  Calls on one stream run in order and can share one
    workspace; calls on two streams get two.  The tensor is allocated with
    that stream current, so when a larger one replaces it, the caching
    allocator hands its memory out again only to work ordered after the
    stream's earlier kernels."""
    s = _stream(device, stream)
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, s.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def ssd_chunk_scan_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, D: torch.Tensor, init_state: Optional[torch.Tensor] = None,
                       chunk_size: int = 256, *, y: Optional[torch.Tensor] = None,
                       final_state: Optional[torch.Tensor] = None, return_final: bool = True,
                       workspace_tensor: Optional[torch.Tensor] = None, algo: str = "auto",
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked SSD scan.  Shapes: x [B,L,H,P], dt [B,L,H] f32, A [H] f32,
    Bm/Cm [B,L,G,N], D [H] f32, init_state [B,H,P,N] f32 or None.
    Returns (y [B,L,H,P], final_state [B,H,P,N] f32 or None)."""
    lib = load_library()
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    _need(x, "x", x.dtype, (Bsz, L, H, P), dev)
    _need(dt, "dt", torch.float32, (Bsz, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(Bm, "Bm", x.dtype, (Bsz, L, G, N), dev)
    _need(Cm, "Cm", x.dtype, (Bsz, L, G, N), dev)
    _need(D, "D", torch.float32, (H,), dev)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (Bsz, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, (Bsz, L, H, P), dev)
    if final_state is None and return_final:
        final_state = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (Bsz, H, P, N), dev)
    code = _dtype_code(x.dtype)
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}")
    need = int(lib.ssd_chunk_scan_workspace_size_algo(Bsz, L, H, P, G, N, chunk_size, code, ALGOS[algo]))
    if workspace_tensor is None:
        workspace_tensor = workspace(need, dev, stream) if need > 0 else None
    ws_bytes = 0 if workspace_tensor is None else workspace_tensor.numel() * workspace_tensor.element_size()
    st = lib.ssd_chunk_scan_fwd_algo(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y),
        _ptr(final_state), _ptr(workspace_tensor), ws_bytes, Bsz, L, H, P, G, N, chunk_size, code,
        ALGOS[algo], _stream_handle(dev, stream))
    _check(st, "ssd_chunk_scan_fwd")
    return y, final_state


def ssd_chunk_scan_fwd_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                               Cm: torch.Tensor, D: torch.Tensor, init_state: Optional[torch.Tensor],
                               chunk_size: int, y: torch.Tensor, final_state: Optional[torch.Tensor] = None, *,
                               stream=None) -> None:
    """The forward scan with the library's static per-device scratch: no
    workspace, and nothing allocated here or in the library.  The caller
    passes y (and final_state, or None to skip it).  Calls on one device
    share the scratch and must not overlap.  Raises SSDError with status
    SSD_ERR_TOO_LARGE for shapes whose workspace exceeds the scratch."""
    lib = load_library()
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    _need(x, "x", x.dtype, (Bsz, L, H, P), dev)
    _need(dt, "dt", torch.float32, (Bsz, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(Bm, "Bm", x.dtype, (Bsz, L, G, N), dev)
    _need(Cm, "Cm", x.dtype, (Bsz, L, G, N), dev)
    _need(D, "D", torch.float32, (H,), dev)
    _need(y, "y", x.dtype, (Bsz, L, H, P), dev)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (Bsz, H, P, N), dev)
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, (Bsz, H, P, N), dev)
    st = lib.ssd_chunk_scan_fwd_noalloc(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y), _ptr(final_state),
        Bsz, L, H, P, G, N, chunk_size, _dtype_code(x.dtype), _stream_handle(dev, stream))
    _check(st, "ssd_chunk_scan_fwd_noalloc")


def ssd_chunk_scan_fwd_varlen(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                              Cm: torch.Tensor, D: torch.Tensor, seq_idx: torch.Tensor,
                              init_state: Optional[torch.Tensor] = None, chunk_size: int = 256, *,
                              y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                              return_final: bool = True, workspace_tensor: Optional[torch.Tensor] = None,
                              stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked SSD scan of packed rows: seq_idx [B,L] int32 names the sequence
    of every token and the state resets where it changes.  Other shapes as
    ssd_chunk_scan_fwd.  Returns (y, final_state of each row's last sequence)."""
    lib = load_library()
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    _need(x, "x", x.dtype, (Bsz, L, H, P), dev)
    _need(dt, "dt", torch.float32, (Bsz, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(Bm, "Bm", x.dtype, (Bsz, L, G, N), dev)
    _need(Cm, "Cm", x.dtype, (Bsz, L, G, N), dev)
    _need(D, "D", torch.float32, (H,), dev)
    _need(seq_idx, "seq_idx", torch.int32, (Bsz, L), dev)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (Bsz, H, P, N), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, (Bsz, L, H, P), dev)
    if final_state is None and return_final:
        final_state = torch.empty((Bsz, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, (Bsz, H, P, N), dev)
    code = _dtype_code(x.dtype)
    need = int(lib.ssd_chunk_scan_varlen_workspace_size(Bsz, L, H, P, G, N, chunk_size, code))
    if workspace_tensor is None:
        workspace_tensor = workspace(need, dev, stream) if need > 0 else None
    ws_bytes = 0 if workspace_tensor is None else workspace_tensor.numel() * workspace_tensor.element_size()
    st = lib.ssd_chunk_scan_fwd_varlen(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(seq_idx), _ptr(y),
        _ptr(final_state), _ptr(workspace_tensor), ws_bytes, Bsz, L, H, P, G, N, chunk_size, code,
        _stream_handle(dev, stream))
    _check(st, "ssd_chunk_scan_fwd_varlen")
    return y, final_state


def ssd_block_prologue(zxbcdt: torch.Tensor, conv_w: torch.Tensor, conv_b: Optional[torch.Tensor],
                       dt_bias: Optional[torch.Tensor], H: int, P: int, G: int, N: int, *,
                       stream=None) -> Dict[str, torch.Tensor]:
    """Split of the block's projection output zxbcdt [B, L, 2HP + 2GN + H]
    (bfloat16), causal depthwise convolution (conv_w [HP + 2GN, W] f32,
    conv_b [HP + 2GN] f32 or None) + SiLU into x [B,L,H,P], Bm, Cm [B,L,G,N],
    and dt = softplus(dt_raw + dt_bias) [B,L,H] f32.  Returns a dict with
    those and z, a view of zxbcdt (no copy)."""
    lib = load_library()
    if zxbcdt.dim() != 3:
        raise ValueError("zxbcdt must be [B, L, 2HP + 2GN + H]")
    Bsz, L, row = zxbcdt.shape
    HP, GN = H * P, G * N
    dev = zxbcdt.device
    _need(zxbcdt, "zxbcdt", torch.bfloat16, (Bsz, L, 2 * HP + 2 * GN + H), dev)
    W = conv_w.shape[1] if conv_w.dim() == 2 else -1
    _need(conv_w, "conv_w", torch.float32, (HP + 2 * GN, W), dev)
    if conv_b is not None:
        _need(conv_b, "conv_b", torch.float32, (HP + 2 * GN,), dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", torch.float32, (H,), dev)
    out = {"x": torch.empty((Bsz, L, H, P), dtype=torch.bfloat16, device=dev),
           "Bm": torch.empty((Bsz, L, G, N), dtype=torch.bfloat16, device=dev),
           "Cm": torch.empty((Bsz, L, G, N), dtype=torch.bfloat16, device=dev),
           "dt": torch.empty((Bsz, L, H), dtype=torch.float32, device=dev)}
    st = lib.ssd_block_prologue(_ptr(zxbcdt), _ptr(conv_w), _ptr(conv_b), _ptr(dt_bias), _ptr(out["x"]),
                                _ptr(out["Bm"]), _ptr(out["Cm"]), _ptr(out["dt"]), Bsz, L, H, P, G, N, W,
                                SSD_DTYPE_BF16, _stream_handle(dev, stream))
    _check(st, "ssd_block_prologue")
    out["z"] = zxbcdt[:, :, :HP]
    return out


def ssd_gated_norm(y: torch.Tensor, z: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                   ngroups: int = 1, eps: float = 1e-5, center: bool = True, *,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gate and group norm of T tokens of D channels: z [..., D] (bfloat16,
    last dimension contiguous; rows may be strided, e.g. the z slice of the
    projection output) and y holding T*D values contiguously (e.g. the scan's
    [B, L, H, P] output for D = H*P).  Returns out shaped like y."""
    lib = load_library()
    D = z.shape[-1]
    T = z.numel() // D if D else 0
    dev = y.device
    if y.dtype != torch.bfloat16 or z.dtype != torch.bfloat16:
        raise TypeError("y and z must be bfloat16")
    if not y.is_contiguous() or y.numel() != T * D:
        raise ValueError("y must be contiguous and hold as many values as z")
    z2 = z.reshape(T, D) if z.dim() != 2 else z
    if z2.stride(1) != 1:
        raise ValueError("z must have a contiguous last dimension")
    zstride = z2.stride(0) if T > 1 else D
    if z.dim() == 3 and T > 1 and z.stride(0) != z.shape[1] * z.stride(1):
        raise ValueError("z rows must be evenly strided")
    _need(weight, "weight", torch.float32, (D,), dev)
    if bias is not None:
        _need(bias, "bias", torch.float32, (D,), dev)
    if out is None:
        out = torch.empty_like(y)
    st = lib.ssd_gated_norm(_ptr(y), _ptr(z2), zstride, _ptr(weight), _ptr(bias), _ptr(out), T, D, ngroups,
                            float(eps), 1 if center else 0, SSD_DTYPE_BF16, _stream_handle(dev, stream))
    _check(st, "ssd_gated_norm")
    return out


def ssd_selective_scan(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor, Cm: torch.Tensor,
                       D: Optional[torch.Tensor] = None, init_state: Optional[torch.Tensor] = None, *,
                       zoh: bool = True, return_final: bool = True,
                       stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Mamba-1 selective scan: x, dt [B, L, Dch] bfloat16, A [Dch, N] f32,
    Bm, Cm [B, L, G, N] bfloat16, D [Dch] f32 or None, init_state
    [B, Dch, N] f32 or None.  Returns (y [B, L, Dch], final_state)."""
    lib = load_library()
    if x.dim() != 3 or Bm.dim() != 4:
        raise ValueError("x must be [B, L, Dch] and Bm [B, L, G, N]")
    Bsz, L, Dch = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    _need(x, "x", torch.bfloat16, (Bsz, L, Dch), dev)
    _need(dt, "dt", torch.bfloat16, (Bsz, L, Dch), dev)
    _need(A, "A", torch.float32, (Dch, N), dev)
    _need(Bm, "Bm", torch.bfloat16, (Bsz, L, G, N), dev)
    _need(Cm, "Cm", torch.bfloat16, (Bsz, L, G, N), dev)
    if D is not None:
        _need(D, "D", torch.float32, (Dch,), dev)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (Bsz, Dch, N), dev)
    y = torch.empty_like(x)
    final = torch.empty((Bsz, Dch, N), dtype=torch.float32, device=dev) if return_final else None
    st = lib.ssd_selective_scan(_ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(y),
                                _ptr(final), Bsz, L, Dch, G, N, 1 if zoh else 0, SSD_DTYPE_BF16,
                                _stream_handle(dev, stream))
    _check(st, "ssd_selective_scan")
    return y, final


def ssd_step(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
             Bm: torch.Tensor, Cm: torch.Tensor, D: torch.Tensor, *,
             y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode token.  state [B,H,P,N] f32 (updated in place), x [B,H,P],
    dt [B,H] f32, A [H] f32, Bm/Cm [B,G,N], D [H] f32.  Returns y [B,H,P]."""
    lib = load_library()
    Bsz, H, P, N = state.shape
    G = Bm.shape[1]
    dev = state.device
    _need(state, "state", torch.float32, (Bsz, H, P, N), dev)
    _need(x, "x", x.dtype, (Bsz, H, P), dev)
    _need(dt, "dt", torch.float32, (Bsz, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(Bm, "Bm", x.dtype, (Bsz, G, N), dev)
    _need(Cm, "Cm", x.dtype, (Bsz, G, N), dev)
    _need(D, "D", torch.float32, (H,), dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, (Bsz, H, P), dev)
    st = lib.ssd_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(y),
                      Bsz, H, P, G, N, _dtype_code(x.dtype), _stream_handle(dev, stream))
    _check(st, "ssd_step")
    return y


def ssd_chunk_scan_varlen_workspace_size(B: int, L: int, H: int, P: int, G: int, N: int,
                                         chunk_size: int, dtype: torch.dtype) -> int:
    return int(load_library().ssd_chunk_scan_varlen_workspace_size(B, L, H, P, G, N, chunk_size,
                                                                   _dtype_code(dtype)))


def ssd_chunk_scan_bwd_workspace_size(B: int, L: int, H: int, P: int, G: int, N: int,
                                      chunk_size: int, dtype: torch.dtype) -> int:
    return int(load_library().ssd_chunk_scan_bwd_workspace_size(B, L, H, P, G, N, chunk_size,
                                                                _dtype_code(dtype)))


def ssd_chunk_scan_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, Bm: torch.Tensor,
                       Cm: torch.Tensor, D: torch.Tensor, init_state: Optional[torch.Tensor],
                       dy: torch.Tensor, dfinal: Optional[torch.Tensor] = None, chunk_size: int = 256, *,
                       want_dinit: bool = True, workspace_tensor: Optional[torch.Tensor] = None,
                       stream=None) -> Dict[str, Optional[torch.Tensor]]:
    """Gradients of <dy, y> + <dfinal, final_state> of the chunk scan with
    respect to x, dt, A, Bm, Cm, D and init_state.  Shapes as
    ssd_chunk_scan_fwd; dy like x, dfinal [B,H,P,N] f32 or None.  Returns a dict
    dx, ddt, dA, dBm, dCm, dD, dinit (dinit None unless want_dinit)."""
    lib = load_library()
    if x.dim() != 4 or Bm.dim() != 4:
        raise ValueError("x must be [B,L,H,P] and Bm [B,L,G,N]")
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    dev = x.device
    _need(x, "x", x.dtype, (Bsz, L, H, P), dev)
    _need(dt, "dt", torch.float32, (Bsz, L, H), dev)
    _need(A, "A", torch.float32, (H,), dev)
    _need(Bm, "Bm", x.dtype, (Bsz, L, G, N), dev)
    _need(Cm, "Cm", x.dtype, (Bsz, L, G, N), dev)
    _need(D, "D", torch.float32, (H,), dev)
    _need(dy, "dy", x.dtype, (Bsz, L, H, P), dev)
    if init_state is not None:
        _need(init_state, "init_state", torch.float32, (Bsz, H, P, N), dev)
    if dfinal is not None:
        _need(dfinal, "dfinal", torch.float32, (Bsz, H, P, N), dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt),
           "dA": torch.empty((H,), dtype=torch.float32, device=dev),
           "dBm": torch.empty_like(Bm), "dCm": torch.empty_like(Cm),
           "dD": torch.empty((H,), dtype=torch.float32, device=dev),
           "dinit": torch.empty((Bsz, H, P, N), dtype=torch.float32, device=dev) if want_dinit else None}
    code = _dtype_code(x.dtype)
    need = int(lib.ssd_chunk_scan_bwd_workspace_size(Bsz, L, H, P, G, N, chunk_size, code))
    if workspace_tensor is None and need > 0:
        with torch.cuda.stream(_stream(dev, stream)):
            workspace_tensor = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace_tensor is None else workspace_tensor.numel() * workspace_tensor.element_size()
    st = lib.ssd_chunk_scan_bwd(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _ptr(init_state), _ptr(dy), _ptr(dfinal),
        _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dBm"]), _ptr(out["dCm"]),
        _ptr(out["dD"]), _ptr(out["dinit"]), _ptr(workspace_tensor), ws_bytes, Bsz, L, H, P, G, N,
        chunk_size, code, _stream_handle(dev, stream))
    _check(st, "ssd_chunk_scan_bwd")
    return out


def ssd_stream_copy(dst: torch.Tensor, src: torch.Tensor, *, stream=None) -> None:
    """Plain device copy of src into dst (same size in bytes, contiguous): the
    bandwidth reference the benchmark reports the kernels against."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if not (src.is_contiguous() and dst.is_contiguous()) or dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must be contiguous tensors of the same size in bytes")
    st = lib.ssd_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream_handle(src.device, stream))
    _check(st, "ssd_stream_copy")


def version() -> str:
    return load_library().ssd_version().decode()
