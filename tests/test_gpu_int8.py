"""GPU parity of segment_attention over an int8 cache (a byte per value with
an fp32 scale for each token and head: the pages' single-GPU format, "The
4090 preset"; the cache is kept in INT8 while the arithmetic runs in BF16,
"El preset de una GPU").

The kernel dequantises each staged key tile to bf16 (code times its token's
scale) and runs the bf16 path. Reference: the oracle over the values the cache
stores (its own per-token quantisation, checked against the kernels' codes by
the append tests) with fp64 queries; bar: the bf16 bar (max-abs 2e-2,
mean-abs 2e-3, relative L2 1e-2; lse 5e-3, see LSE_ATOL). Raw K and V are
N(0, 1): per-(frame, head) factors would only scale the bar (the int8 scales
are per token). Against exact attention on the
unquantised inputs the storage error is added: relative L2 <= 5e-2.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, compare

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_L2 = 2e-2, 2e-3, 1e-2
# lse: the bf16 path's 4e-3 (bf16-rounded probabilities in the row sum, bf16
# rounding of rotated Q and of the dequantised K) plus the K codes and scales
# that the kernel's fp32 rotation moves from the oracle's (measured on the
# CPU: below 1e-3 of lse)
LSE_ATOL = 5e-3


def _wl(name, H, F, lh, lw, n_text, prior):
    return si.Workload(name, heads=H, lat_t=F, lat_h=lh, lat_w=lw, n_text=n_text,
                       prior_segments=(prior,), kv_dtype="int8")


def _check(s, label, rows=None, heads=None):
    got, got_lse = s.gpu_out(rows=rows, heads=heads)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse)), label
    want, want_lse = s.oracle_int8_cache(rows=rows, heads=heads)
    _, _, rel = compare(got, want, MAX_ABS, MEAN_ABS, label)
    assert rel <= REL_L2, label
    np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0, err_msg=label)
    return got


CASES = [
    # name, H, F, lat_h, lat_w, n_text, prior segments
    ("i8_small", 2, 2, 4, 8, 16, 2),       # P = 32
    ("i8_p24", 2, 3, 4, 6, 16, 2),         # P = 24: planes of 32 token slots
    ("i8_ragged", 3, 5, 4, 8, 37, 3),      # ragged query and text tails
    ("i8_p80", 2, 4, 8, 10, 64, 2),        # frame = 64 + 16 keys
    ("i8_big", 4, 6, 8, 16, 256, 2),       # Lq = 1024, Lk = 2560
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_int8_parity_small(case):
    name, H, F, lh, lw, nt, prior = case
    print(f"int8 attention parity case={name}", flush=True)
    wl = _wl(name, H, F, lh, lw, nt, prior)
    s = Session(wl, seed=111, layer=0, session=0)
    sa.segment_attention(s.geom, [s.item()], workspace=None)
    torch.cuda.synchronize()
    got = _check(s, name)
    want, _ = s.oracle()
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    print(f"{name}: relative L2 against exact attention on unquantised inputs {rel:.3e}", flush=True)
    assert rel <= 5e-2


def test_int8_split_tiles_and_windows():
    """Split parts (workspace) and timed text windows on an int8 cache."""
    wl = _wl("i8_split", 4, 6, 8, 16, 256, 2)
    s = Session(wl, seed=113, layer=0, session=0)
    assert sa.segment_attention_workspace(s.geom, [s.item()]) > 0
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check(s, "int8 split")
    s.set_windows(si.text_windows(wl, 113, s.S * wl.lat_t).numpy())
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check(s, "int8 split + windows")


def test_int8_sparse_history():
    """Block-sparse history on an int8 cache: sparse_select pools the stored
    keys (codes times their token's scale) and the attention walks the kept
    blocks; checked with the oracle's lists, and the GPU lists against them."""
    from helpers import check_block_lists
    wl = _wl("i8_sparse", 2, 4, 8, 16, 40, 3)
    s = Session(wl, seed=115, layer=0, session=0)
    n_hist = 12
    keep = sa.sparse_keep(n_hist * 2, 25)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    got_lists = sa.sparse_select(s.geom, it).cpu().numpy()
    want_lists, scores = s.oracle_select(n_hist, keep)
    check_block_lists(got_lists, want_lists, scores, 1e-3)
    s.set_sparse(want_lists, n_hist)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check(s, "int8 sparse")


def test_int8_eight_prior_segments_two_heads():
    """The int8 workload's shape at one GPU's 2-head share: eight prior
    segments (237,856 keys), sampled rows against the stored-values oracle."""
    wl = si.Workload("i8seg8h2", heads=2, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                     prior_segments=(8,), kv_dtype="int8")
    print("workload int8, eight prior segments, 2 heads", flush=True)
    s = Session(wl, 0, 0, 0)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    v = wl.lat_t * wl.P
    rows = si.sample_rows(wl.Lq, 96, 17, [255, 256, v - 1, v, wl.Lq - 1])
    _check(s, "int8 seg8 2 heads", rows=rows)
