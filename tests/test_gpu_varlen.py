"""GPU parity of ssd_chunk_scan_fwd_varlen (packed rows, state reset at every
sequence boundary) against the fp64 oracle, through the C ABI.

The oracle (oracle/varlen.py) scans every run of equal seq_idx values on its
own.  y and the final state are compared with gpu_util.rel_err at the
bfloat16 limit, 2e-2.  The cases put boundaries on and next to the 64-token
sub-block edges, use one-token sequences, and run the shapes where the
launcher spreads a row over several workgroups in time segments (every
sequence cut; and one whole sequence per workgroup plus segments of the
rest), so that a reset inside a segment is covered.  Every case prints its
name and shape before it touches the GPU.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
from gpu_util import TOL, announce, rel_err, to_device, to_np

from oracle.varlen import recurrence_varlen

pytestmark = pytest.mark.gpu


def _oracle(d, seq, bh=None):
    f = si.as_f64(d)
    return recurrence_varlen(f["x"], f["dt"], f["A"], f["Bm"], f["Cm"], f["D"], f["init"], seq, bh=bh)


def _gpu(dd, seq):
    import selective_state_space_chunk_amd as ssd
    y, fin = ssd.ssd_chunk_scan_fwd_varlen(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"],
                                           torch.from_numpy(seq).to("cuda"), dd["init"])
    torch.cuda.synchronize()
    return y, fin


# (name, B, L, H, N, G, init, lengths (None: random with mean_len), mean_len)
CASES = [
    ("two_docs_one_block", 1, 64, 2, 128, 1, True, [[20, 44]], None),
    ("resets_on_sub_block_edges", 2, 256, 3, 64, 1, True, [[64, 64, 128], [1, 63, 65, 127]], None),
    ("one_token_docs", 1, 150, 2, 128, 1, False, [[1] * 10 + [5, 1, 1, 63, 1, 64]], None),
    ("random_packing_ragged_groups", 2, 1000, 4, 128, 2, True, None, 120.0),
    ("every_sequence_cut_in_segments", 1, 3000, 4, 128, 1, True, None, 300.0),
    ("long_doc_across_segments", 1, 3000, 4, 64, 1, True, [[2000, 1000]], None),
    ("whole_rows_plus_segments", 3, 700, 100, 128, 4, True, None, 90.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_matches_oracle(case):
    name, B, L, H, N, G, init, lengths, mean_len = case
    d = si.make_scan_inputs(B, L, H, 64, N, G, dtype="bf16", init=init, seed=4100 + L + H)
    seq = si.make_seq_idx(B, L, lengths=lengths, mean_len=mean_len or 512.0, seed=4200 + L)
    nseq = [int(seq[b, -1]) + 1 for b in range(B)]
    bh = None if B * H <= 16 else [b * H + h for b in range(B) for h in (0, H // 2, H - 1)]
    y_ref, f_ref = _oracle(d, seq, bh)
    announce(f"varlen {name}: B{B} L{L} H{H} P64 N{N} G{G} init={init} sequences per row {nseq}")
    y, fin = _gpu(to_device(d, "bf16"), seq)
    y, fin = to_np(y), to_np(fin)
    if bh is not None:
        ys = np.stack([y[k // H, :, k % H] for k in bh])
        yr = np.stack([y_ref[k // H, :, k % H] for k in bh])
        fs = np.stack([fin[k // H, k % H] for k in bh])
        fr = np.stack([f_ref[k // H, k % H] for k in bh])
    else:
        ys, yr, fs, fr = y, y_ref, fin, f_ref
    ey, ef = rel_err(ys, yr), rel_err(fs, fr)
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_varlen_head_dim_128():
    # P = 128: every head scanned as two heads of 64 channels sharing dt (and
    # its reset flags); the rows are cut into segments (6 such heads)
    B, L, H, N = 1, 2500, 3, 128
    d = si.make_scan_inputs(B, L, H, 128, N, 1, dtype="bf16", init=True, seed=4701)
    seq = si.make_seq_idx(B, L, mean_len=300.0, seed=4702)
    y_ref, f_ref = _oracle(d, seq)
    announce(f"varlen P128: B{B} L{L} H{H} N{N}, sequences per row {[int(seq[b, -1]) + 1 for b in range(B)]}")
    y, fin = _gpu(to_device(d, "bf16"), seq)
    ey, ef = rel_err(to_np(y), y_ref), rel_err(to_np(fin), f_ref)
    print(f"    y {ey:.3e}  final {ef:.3e}", flush=True)
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (ey, ef)


def test_varlen_full_size_sampled_heads():
    # the Mamba-2 2.7B layer shape with documents packed into each row
    B, L, H, N = 4, 4096, 80, 128
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=4301)
    seq = si.make_seq_idx(B, L, mean_len=512.0, seed=4302)
    bh = [0 * H + 0, 1 * H + 41, 2 * H + 79, 3 * H + 17]
    y_ref, f_ref = _oracle(d, seq, bh)
    announce(f"varlen full size: B{B} L{L} H{H} N{N}, sequences per row {[int(seq[b, -1]) + 1 for b in range(B)]}")
    y, fin = _gpu(to_device(d, "bf16"), seq)
    y, fin = to_np(y), to_np(fin)
    for k in bh:
        b, h = divmod(k, H)
        ey, ef = rel_err(y[b, :, h], y_ref[b, :, h]), rel_err(fin[b, h], f_ref[b, h])
        print(f"    b{b} h{h}: y {ey:.3e} final {ef:.3e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (k, ey, ef)


def test_no_boundaries_equal_the_plain_scan():
    import selective_state_space_chunk_amd as ssd
    B, L, H, N = 1, 3000, 4, 128          # segmented launch
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=4401)
    dd = to_device(d, "bf16")
    announce(f"varlen without boundaries vs the plain scan: B{B} L{L} H{H} N{N}")
    y0, f0 = ssd.ssd_chunk_scan_fwd(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["D"], dd["init"])
    y1, f1 = _gpu(dd, np.zeros((B, L), dtype=np.int32))
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


def test_varlen_without_tokens():
    import selective_state_space_chunk_amd as ssd
    H, N = 3, 64
    init = torch.randn(2, H, 64, N, device="cuda")
    x = torch.empty((2, 0, H, 64), dtype=torch.bfloat16, device="cuda")
    Bm = torch.empty((2, 0, 1, N), dtype=torch.bfloat16, device="cuda")
    announce("varlen with L = 0")
    _, fin = ssd.ssd_chunk_scan_fwd_varlen(x, torch.empty((2, 0, H), device="cuda"), torch.full((H,), -1.0, device="cuda"),
                                           Bm, Bm.clone(), torch.ones(H, device="cuda"),
                                           torch.empty((2, 0), dtype=torch.int32, device="cuda"), init)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)


def test_varlen_rejects_uncovered_shapes():
    import selective_state_space_chunk_amd as ssd
    d = si.make_scan_inputs(1, 70, 2, 32, 64, 1, dtype="bf16", seed=4501)
    dd = to_device(d, "bf16")
    announce("varlen P=32 is not covered")
    with pytest.raises(ssd.SSDError) as ei:
        _gpu(dd, np.zeros((1, 70), dtype=np.int32))
    assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED


def test_varlen_at_the_130m_shape_sampled_heads():
    # the Mamba-2 130M layer shape (B 8, L 2048, H 24: 192 sequences, one workgroup each)
    B, L, H, N = 8, 2048, 24, 128
    d = si.make_scan_inputs(B, L, H, 64, N, 1, dtype="bf16", init=True, seed=4601)
    seq = si.make_seq_idx(B, L, mean_len=256.0, seed=4602)
    bh = [0 * H + 0, 3 * H + 12, 7 * H + 23]
    y_ref, f_ref = _oracle(d, seq, bh)
    announce(f"varlen at the 130M shape: B{B} L{L} H{H} N{N}, sampled heads")
    y, fin = _gpu(to_device(d, "bf16"), seq)
    y, fin = to_np(y), to_np(fin)
    for k in bh:
        b, h = divmod(k, H)
        ey, ef = rel_err(y[b, :, h], y_ref[b, :, h]), rel_err(fin[b, h], f_ref[b, h])
        print(f"    b{b} h{h}: y {ey:.3e} final {ef:.3e}", flush=True)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (k, ey, ef)
