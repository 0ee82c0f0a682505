"""GPU parity on the five workloads at their full sizes (through the C ABI).

Each workload is built exactly as the bench builds it (same seeded inputs, the
same kv_append / text_append / segment_attention calls and launch shapes); the
oracle recomputes a seeded sample of query rows one by one from the raw
inputs: the first and last rows, the rows on both sides of every 128-row
workgroup boundary near the video/text split, the first and last text rows,
and random rows. Gate: max-abs <= 2e-2, mean-abs <= 2e-3 and relative L2
<= 1e-2 for a bf16 cache; the e4m3 cache as its test states.
"""

import gc

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists, compare

pytestmark = pytest.mark.gpu

WL = {w.name: w for w in si.workloads(0)}
# lse: bf16-rounded probabilities in the row sum (2^-9 relative) plus the
# bf16 rounding of rotated Q and K.
LSE_ATOL = 4e-3


def _rows(wl, n, seed):
    v = wl.lat_t * wl.P
    bounds = [127, 128, 255, 256, v - 129, v - 128, v - 1, v, v + 1, wl.Lq - 2, wl.Lq - 1,
              wl.P - 1, wl.P, 2 * wl.P]
    return si.sample_rows(wl.Lq, n, seed, bounds)


def _check(sessions, n_rows, heads=None, tol=(2e-2, 2e-3, 1e-2), label=""):
    for s in sessions:
        rows = _rows(s.wl, n_rows, s.session + 11)
        want, want_lse = s.oracle(rows=rows, heads=heads)
        got, got_lse = s.gpu_out(rows=rows, heads=heads)
        _, _, rel = compare(got, want, tol[0], tol[1], f"{label} session {s.session}")
        assert rel <= tol[2]
        np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0)


def test_tiny_full_output():
    wl = WL["tiny"]
    s = Session(wl, 0, 0, 0)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    want, want_lse = s.oracle()
    got, got_lse = s.gpu_out()
    compare(got, want, 2e-2, 2e-3, "tiny")
    np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0)


def test_one_prior_segment():
    wl = WL["seg1"]
    print("workload seg1: 26,656 queries x 53,056 keys x 16 heads", flush=True)
    s = Session(wl, 0, 0, 0)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check([s], 192, label="seg1")


def test_one_prior_segment_two_heads():
    """One GPU's share of the one-prior-segment workload when the 16 heads are
    spread over 8 GPUs: 2 heads, 210 query tiles, fewer than the compute
    units, so every tile runs as key-range parts merged afterwards."""
    wl = si.Workload("seg1h2", heads=2, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                     prior_segments=(1,))
    print("workload seg1 at 2 heads: 26,656 queries x 53,056 keys", flush=True)
    s = Session(wl, 0, 0, 0)
    assert sa.segment_attention_workspace(s.geom, [s.item()]) > 0
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check([s], 192, label="seg1 2 heads")


def test_long_history_54_layers():
    """Four prior segments, 54 independent seeded layers: every layer checked on
    a row sample over two heads; layers 0 and 53 on all heads."""
    wl = WL["seg4x54"]
    for layer in range(wl.layers):
        print(f"workload seg4x54 layer {layer}", flush=True)
        s = Session(wl, 0, layer, 0)
        sa.segment_attention(s.geom, [s.item()])
        torch.cuda.synchronize()
        if layer in (0, wl.layers - 1):
            _check([s], 96, label=f"seg4x54 layer {layer}")
        else:
            heads = [layer % wl.heads, (7 * layer + 3) % wl.heads]
            _check([s], 24, heads=sorted(set(heads)), label=f"seg4x54 layer {layer}")
        del s
        gc.collect()
        torch.cuda.empty_cache()


def test_active_history_selection_two_sessions():
    wl = WL["select2"]
    print(f"workload select2: prior segments {wl.prior_segments}", flush=True)
    ss = [Session(wl, 0, 0, i) for i in range(2)]
    assert len(ss[0].frames) == 99 + 30
    sa.segment_attention(ss[0].geom, [s.item() for s in ss])
    torch.cuda.synchronize()
    _check(ss, 128, label="select2")


def test_fp8_cache_eight_prior_segments():
    """Eight prior segments stored e4m3 with per-(frame, head) scales; values
    scaled by U[0.5, 2] per (frame, head); 237,856 keys.

    The cache bytes are bit-exact to the oracle's quantisation (append tests),
    so the kernel is gated against the oracle over the values the cache stores,
    at 2e-2 / 2e-3. Against exact attention on the unquantised inputs the
    error includes storing K and V in e4m3, which the oracle measures itself
    on the same rows: max-abs within that storage error + 2e-2, mean-abs
    within 5e-3, relative L2 within 0.1. (With these inputs the storage error
    alone reaches about 5e-2 at the worst sampled element.)"""
    wl = WL["fp8seg8"]
    print("workload fp8seg8: 26,656 queries x 237,856 keys x 16 heads", flush=True)
    s = Session(wl, 0, 0, 0)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    rows = _rows(wl, 48, 3)
    heads = [0, 5, 11, 15]
    got, got_lse = s.gpu_out(rows=rows, heads=heads)
    want_c, want_c_lse, _ = s.oracle_fp8_cache(rows=rows, heads=heads)
    _, _, rel = compare(got, want_c, 2e-2, 2e-3, "fp8seg8 vs stored cache")
    assert rel <= 0.05
    np.testing.assert_allclose(got_lse, want_c_lse, atol=2e-2, rtol=0)
    want, _ = s.oracle(rows=rows, heads=heads)
    storage = float(np.max(np.abs(want_c - want)))
    print(f"fp8seg8: e4m3 storage error of the oracle itself {storage:.3e}", flush=True)
    _, _, rel = compare(got, want, storage + 2e-2, 5e-3, "fp8seg8 vs exact")
    assert rel <= 0.1


def test_sparse_history_four_prior_segments_two_heads():
    """Block-sparse history at full size on one GPU's 2-head share of the
    four-prior-segment workload: 120 history frames (1,680 candidate blocks,
    420 kept) for 105 query blocks. sparse_select is checked on every list
    against the oracle's selection (equal up to near-ties at the threshold);
    the attention runs with the oracle's lists and is checked on sampled rows
    against the oracle's sparse attention."""
    wl = si.Workload("seg4h2", heads=2, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                     prior_segments=(4,))
    print("workload seg4 at 2 heads, block-sparse history (25 %)", flush=True)
    s = Session(wl, 0, 0, 0)
    n_hist = 4 * 30
    keep = sa.sparse_keep(n_hist * 14, 25)
    assert keep == 420
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    got_lists = sa.sparse_select(s.geom, it).cpu().numpy()
    want_lists, scores = s.oracle_select(n_hist, keep)
    swaps = check_block_lists(got_lists, want_lists, scores, 1e-4)
    print(f"near-tie swaps: {swaps} of {want_lists.size} list entries", flush=True)
    s.set_sparse(want_lists, n_hist)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check([s], 192, label="seg4 2 heads sparse")
