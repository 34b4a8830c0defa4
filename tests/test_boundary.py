"""Host-only checks of the C ABI: the library loads, exports every entry point
include/libssd.h declares, sizes workspaces, and rejects bad arguments before
anything reaches the GPU.  No call here launches a kernel: every call either
is a pure host query or returns an error status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libssd.h")


@pytest.fixture(scope="module")
def lib():
    import selective_state_space_chunk_amd as ssd
    if not os.path.exists(ssd.LIB_PATH):
        from selective_state_space_chunk_amd import build
        build.build()
    return ssd.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssd_chunk_scan_fwd", "ssd_step", "ssd_chunk_scan_workspace_size",
              "ssd_status_string", "ssd_chunk_scan_fwd_algo", "ssd_version",
              "ssd_chunk_scan_workspace_size_algo", "ssd_chunk_scan_bwd", "ssd_chunk_scan_bwd_workspace_size",
              "ssd_chunk_scan_fwd_varlen", "ssd_chunk_scan_varlen_workspace_size", "ssd_block_prologue",
              "ssd_gated_norm", "ssd_selective_scan", "ssd_chunk_scan_fwd_noalloc", "ssd_stream_copy"):
        assert n in names


def test_noalloc_scratch_size_matches_the_binding():
    import selective_state_space_chunk_amd as ssd
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == ssd.NOALLOC_SCRATCH_BYTES


def test_library_exports_every_declared_symbol(lib):
    import selective_state_space_chunk_amd as ssd
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings_and_version(lib):
    import selective_state_space_chunk_amd as ssd
    for code in range(6):
        assert ssd.status_string(code).startswith("SSD_")
    assert "gfx950" in ssd.version()


B, L, H, P, G, N, Q = 4, 4096, 80, 64, 1, 128, 256


def align(v):
    return (v + 255) // 256 * 256


def test_workspace_size(lib):
    AUTO, REFERENCE, STAGED, PIPE = 0, 1, 2, 3
    # the per-sequence scan (what AUTO runs here): the gram tiles of every
    # 64-token sub-block and room for 256 segment states, nothing per block
    ws = lib.ssd_chunk_scan_workspace_size(B, L, H, P, G, N, Q, 1)
    gram = B * G * (L // 64) * 64 * 64 * 2
    seg = 256 * (P * N + 1) * 4
    assert ws == align(seg) + align(gram)
    assert ws == lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 1, PIPE)
    assert ws == lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 1, AUTO)
    # the staged and reference forms keep every block's state and decay
    nc = L // Q
    states = align(B * nc * H * P * N * 4) + align(B * H * nc * 4)
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 1, STAGED) == states + align(gram)
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 1, REFERENCE) == states
    # N = 256 runs the per-sequence scan under AUTO too; float32 runs the reference
    assert lib.ssd_chunk_scan_workspace_size(1, 1000, 4, P, 1, 256, 128, 1) == \
        lib.ssd_chunk_scan_workspace_size_algo(1, 1000, 4, P, 1, 256, 128, 1, PIPE) == \
        align(4 * 15 * (P * 256 + 1) * 4) + align(16 * 8192)
    assert lib.ssd_chunk_scan_workspace_size(1, 1000, 4, P, 1, 128, 128, 0) == \
        lib.ssd_chunk_scan_workspace_size_algo(1, 1000, 4, P, 1, 128, 128, 0, REFERENCE)
    # a short sequence is cut into at most its sub-blocks: two sub-blocks, one segment state
    assert lib.ssd_chunk_scan_workspace_size(1, 128, 1, P, 1, N, Q, 1) == align((P * N + 1) * 4) + align(2 * 8192)
    # ragged L rounds the sub-block count up
    assert lib.ssd_chunk_scan_workspace_size(B, L + 1, H, P, G, N, Q, 1) > ws
    # unsupported shapes, dtypes and algorithms report 0
    for bad in [(B, L, H, 48, G, N, Q), (B, L, H, P, G, 512, Q), (B, L, H, P, G, N, 32),
                (B, L, H, P, 3, N, Q), (-1, L, H, P, G, N, Q)]:
        assert lib.ssd_chunk_scan_workspace_size(*bad, 1) == 0
    assert lib.ssd_chunk_scan_workspace_size(B, L, H, P, G, N, Q, 7) == 0
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 1, 9) == 0
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, P, G, N, Q, 0, PIPE) == 0      # float32
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, 32, G, N, Q, 1, STAGED) == 0   # P = 32
    assert lib.ssd_chunk_scan_workspace_size_algo(B, L, H, 128, G, N, Q, 1, STAGED) == 0  # P = 128
    # P = 128 runs the per-sequence scan as twice the heads of 64 channels
    assert lib.ssd_chunk_scan_workspace_size(2, 640, 3, 128, 1, N, Q, 1) == \
        align(2 * 6 * 9 * (64 * N + 1) * 4) + align(2 * 10 * 8192)


def fake(addr):
    return ctypes.c_void_p(addr)


def scan_call(lib, *, x=0x10000, dt=0x20000, A=0x30000, Bm=0x40000, Cm=0x50000, D=0x60000,
              init=None, y=0x70000, fin=None, ws=0x80000, ws_bytes=None, shape=(B, L, H, P, G, N, Q),
              dtype=1, algo=0):
    b, l, h, p, g, n, q = shape
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.ssd_chunk_scan_fwd_algo(fake(x) if x else None, fake(dt) if dt else None,
                                       fake(A) if A else None, fake(Bm) if Bm else None,
                                       fake(Cm) if Cm else None, fake(D) if D else None,
                                       fake(init) if init else None, fake(y) if y else None,
                                       fake(fin) if fin else None, fake(ws) if ws else None,
                                       ws_bytes, b, l, h, p, g, n, q, dtype, algo, None)


def test_scan_rejects_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd
    assert scan_call(lib, x=0) == ssd.SSD_ERR_INVALID_ARG            # null input
    assert scan_call(lib, y=0) == ssd.SSD_ERR_INVALID_ARG            # null output
    assert scan_call(lib, Bm=0x40008) == ssd.SSD_ERR_INVALID_ARG     # misaligned
    assert scan_call(lib, init=0x90004) == ssd.SSD_ERR_INVALID_ARG   # misaligned init
    assert scan_call(lib, shape=(B, -1, H, P, G, N, Q)) == ssd.SSD_ERR_INVALID_ARG
    assert scan_call(lib, shape=(B, L, H, P, 3, N, Q)) == ssd.SSD_ERR_INVALID_ARG   # H % G
    assert scan_call(lib, shape=(B, L, H, P, G, N, 0)) == ssd.SSD_ERR_INVALID_ARG
    assert scan_call(lib, shape=(B, L, H, 48, G, N, Q)) == ssd.SSD_ERR_UNSUPPORTED
    assert scan_call(lib, shape=(B, L, H, P, G, 512, Q)) == ssd.SSD_ERR_UNSUPPORTED
    assert scan_call(lib, shape=(B, L, H, P, G, N, 32)) == ssd.SSD_ERR_UNSUPPORTED
    assert scan_call(lib, dtype=5) == ssd.SSD_ERR_UNSUPPORTED
    assert scan_call(lib, algo=9) == ssd.SSD_ERR_UNSUPPORTED
    # matrix-core algorithms need bf16 and P = 64
    assert scan_call(lib, dtype=0, algo=3) == ssd.SSD_ERR_UNSUPPORTED
    assert scan_call(lib, shape=(B, L, H, 32, G, N, Q), algo=2) == ssd.SSD_ERR_UNSUPPORTED
    # workspace missing or too small, for the algorithm the call runs
    assert scan_call(lib, ws=0) == ssd.SSD_ERR_WORKSPACE
    need = lib.ssd_chunk_scan_workspace_size(B, L, H, P, G, N, Q, 1)
    assert scan_call(lib, ws_bytes=need - 1) == ssd.SSD_ERR_WORKSPACE
    assert scan_call(lib, ws_bytes=need, algo=2) == ssd.SSD_ERR_WORKSPACE   # staged needs its block states


def test_step_rejects_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd

    def call(state=0x1000, x=0x2000, shape=(256, 80, 64, 1, 128), dtype=1):
        b, h, p, g, n = shape
        return lib.ssd_step(fake(state) if state else None, fake(x) if x else None, fake(0x3000),
                            fake(0x4000), fake(0x5000), fake(0x6000), fake(0x7000), fake(0x8000),
                            b, h, p, g, n, dtype, None)
    assert call(state=0) == ssd.SSD_ERR_INVALID_ARG
    assert call(x=0) == ssd.SSD_ERR_INVALID_ARG
    assert call(state=0x1004) == ssd.SSD_ERR_INVALID_ARG
    assert call(shape=(256, 80, 64, 3, 128)) == ssd.SSD_ERR_INVALID_ARG
    assert call(shape=(256, 80, 64, 1, 512)) == ssd.SSD_ERR_UNSUPPORTED
    assert call(shape=(256, 80, 48, 1, 128)) == ssd.SSD_ERR_UNSUPPORTED
    assert call(dtype=3) == ssd.SSD_ERR_UNSUPPORTED
    assert call(shape=(0, 80, 64, 1, 128)) == ssd.SSD_OK                 # empty batch: no-op


def test_stream_copy_rejects_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd
    assert lib.ssd_stream_copy(fake(0x10000), fake(0x20000), 0, None) == ssd.SSD_OK          # nothing to copy
    assert lib.ssd_stream_copy(None, fake(0x20000), 16, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_stream_copy(fake(0x10008), fake(0x20000), 16, None) == ssd.SSD_ERR_INVALID_ARG   # misaligned
    assert lib.ssd_stream_copy(fake(0x10000), fake(0x20000), 24, None) == ssd.SSD_ERR_INVALID_ARG   # not 16-byte units
    assert lib.ssd_stream_copy(fake(0x10000), fake(0x10100), 4096, None) == ssd.SSD_ERR_INVALID_ARG  # overlapping


def test_binding_refuses_to_run_without_library(monkeypatch):
    import selective_state_space_chunk_amd as ssd
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "LIB_PATH", "/nonexistent/libssd.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        ssd.load_library()


def test_backward_workspace_size(lib):
    # states entering and gradients leaving every sub-block: two bfloat16 arrays of
    # B*H*nsb*64*N, plus B*H*nsb float32 parts of dA and of dD
    nsb = (L + 63) // 64
    want = 2 * 2 * B * H * nsb * 64 * N + 4 * 2 * B * H * nsb
    want = (want + 255) // 256 * 256
    assert lib.ssd_chunk_scan_bwd_workspace_size(B, L, H, P, G, N, Q, 1) == want
    # heads of 128 channels: states of both halves, parts per head
    want = 2 * 2 * B * H * nsb * 128 * N + 4 * 2 * B * H * nsb
    want = (want + 255) // 256 * 256
    assert lib.ssd_chunk_scan_bwd_workspace_size(B, L, H, 128, G, N, Q, 1) == want
    # not covered: float32, P not 64 or 128, N = 256
    assert lib.ssd_chunk_scan_bwd_workspace_size(B, L, H, P, G, N, Q, 0) == 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(B, L, H, 32, G, N, Q, 1) == 0
    assert lib.ssd_chunk_scan_bwd_workspace_size(B, L, H, P, G, 256, Q, 1) == 0


def test_varlen_rejects_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd

    def call(x=0x10000, seq=0x90000, ws=0x80000, ws_bytes=1 << 40, shape=(B, L, H, P, G, N, Q), dtype=1):
        b, l, h, p, g, n, q = shape
        return lib.ssd_chunk_scan_fwd_varlen(fake(x) if x else None, fake(0x20000), fake(0x30000), fake(0x40000),
                                             fake(0x50000), fake(0x60000), None, fake(seq) if seq else None,
                                             fake(0x70000), None, fake(ws) if ws else None, ws_bytes,
                                             b, l, h, p, g, n, q, dtype, None)
    assert call(x=0) == ssd.SSD_ERR_INVALID_ARG
    assert call(seq=0) == ssd.SSD_ERR_INVALID_ARG                    # no sequence index
    assert call(seq=0x90002) == ssd.SSD_ERR_INVALID_ARG              # misaligned int32
    assert call(shape=(B, L, H, P, G, N, 0)) == ssd.SSD_ERR_INVALID_ARG
    assert call(dtype=0) == ssd.SSD_ERR_UNSUPPORTED
    assert call(shape=(B, L, H, 32, G, N, Q)) == ssd.SSD_ERR_UNSUPPORTED
    need = lib.ssd_chunk_scan_varlen_workspace_size(B, L, H, P, G, N, Q, 1)
    assert need >= lib.ssd_chunk_scan_workspace_size(B, L, H, P, G, N, Q, 1) + B * L * H * 4
    assert call(ws=0) == ssd.SSD_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == ssd.SSD_ERR_WORKSPACE


def test_block_steps_reject_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd

    def pro(zx=0x10000, x=0x20000, shape=(4, 4096, 80, 64, 1, 128, 4), dtype=1):
        b, l, h, p, g, n, w = shape
        return lib.ssd_block_prologue(fake(zx) if zx else None, fake(0x30000), None, None, fake(x) if x else None,
                                      fake(0x40000), fake(0x50000), fake(0x60000), b, l, h, p, g, n, w, dtype, None)
    assert pro(zx=0) == ssd.SSD_ERR_INVALID_ARG
    assert pro(x=0x20008) == ssd.SSD_ERR_INVALID_ARG                 # misaligned output
    assert pro(shape=(4, 4096, 80, 64, 3, 128, 4)) == ssd.SSD_ERR_INVALID_ARG      # H % G
    assert pro(shape=(4, 4096, 80, 64, 1, 128, 0)) == ssd.SSD_ERR_INVALID_ARG
    assert pro(shape=(4, 4096, 80, 64, 1, 128, 5)) == ssd.SSD_ERR_UNSUPPORTED      # width 5
    assert pro(shape=(4, 4096, 4, 64, 1, 128, 4)) == ssd.SSD_ERR_UNSUPPORTED       # row not a multiple of 8
    assert pro(dtype=0) == ssd.SSD_ERR_UNSUPPORTED
    assert pro(shape=(0, 4096, 80, 64, 1, 128, 4)) == ssd.SSD_OK                   # nothing to do

    def norm(y=0x10000, w=0x30000, T=16, D=5120, zstride=5120, ngroups=1, eps=1e-5, dtype=1):
        return lib.ssd_gated_norm(fake(y) if y else None, fake(0x20000), zstride, fake(w), None, fake(0x40000),
                                  T, D, ngroups, eps, 1, dtype, None)
    assert norm(y=0) == ssd.SSD_ERR_INVALID_ARG
    assert norm(w=0x30004) == ssd.SSD_ERR_INVALID_ARG                # misaligned weight
    assert norm(eps=-1.0) == ssd.SSD_ERR_INVALID_ARG
    assert norm(ngroups=0) == ssd.SSD_ERR_INVALID_ARG
    assert norm(ngroups=9) == ssd.SSD_ERR_UNSUPPORTED
    assert norm(D=8200, zstride=8200) == ssd.SSD_ERR_UNSUPPORTED     # wider than 8192
    assert norm(zstride=5000) == ssd.SSD_ERR_UNSUPPORTED             # stride below the row
    assert norm(dtype=0) == ssd.SSD_ERR_UNSUPPORTED
    assert norm(T=0) == ssd.SSD_OK


def test_selective_scan_rejects_bad_arguments_before_launch(lib):
    import selective_state_space_chunk_amd as ssd

    def call(x=0x10000, y=0x70000, shape=(4, 4096, 5120, 1, 16), dtype=1):
        b, l, dch, g, n = shape
        return lib.ssd_selective_scan(fake(x) if x else None, fake(0x20000), fake(0x30000), fake(0x40000),
                                      fake(0x50000), None, None, fake(y) if y else None, None,
                                      b, l, dch, g, n, 1, dtype, None)
    assert call(x=0) == ssd.SSD_ERR_INVALID_ARG
    assert call(y=0x70002) == ssd.SSD_ERR_INVALID_ARG
    assert call(shape=(4, 4096, 5120, 3, 16)) == ssd.SSD_ERR_INVALID_ARG   # Dch % G
    assert call(shape=(4, 4096, 5120, 1, 12)) == ssd.SSD_ERR_UNSUPPORTED
    assert call(shape=(4, 4096, 96, 1, 16)) == ssd.SSD_ERR_UNSUPPORTED
    assert call(dtype=0) == ssd.SSD_ERR_UNSUPPORTED
    assert call(shape=(0, 4096, 5120, 1, 16)) == ssd.SSD_OK
