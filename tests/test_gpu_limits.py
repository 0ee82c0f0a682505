"""GPU parity at the limits the C ABI states, against the oracle.

- sparse_select at SA_MAX_SPARSE_CANDIDATES (8,192 candidate blocks: 8,192
  history frames of 64 tokens), the selection kernel's largest radix-select
  and scan, and the attention over its lists;
- block-sparse history whose candidates are only part of the history (the
  other history frames stay dense), and a single kept block;
- timed text windows at the window-table bound: frames of 16 tokens with
  3,616 text keys fill (255 / 16 + 3) * ceil(3616 / 32) = 2,034 of the 2,048
  table words (one more word is refused on the host: tests/test_abi_cpu.py).
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists, compare

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_L2, LSE_ATOL = 2e-2, 2e-3, 1e-2, 4e-3


def _check(s, label, rows=None):
    got, got_lse = s.gpu_out(rows=rows)
    want, want_lse = s.oracle(rows=rows)
    _, _, rel = compare(got, want, MAX_ABS, MEAN_ABS, label)
    assert rel <= REL_L2, label
    np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0, err_msg=label)


def test_select_at_the_candidate_bound():
    """8,192 candidates (128 prior segments of 64 frames of 8 x 8 tokens: one
    block per frame), one head, 17 query blocks; keep 2,048."""
    wl = si.Workload("maxcand", heads=1, lat_t=64, lat_h=8, lat_w=8, n_text=16,
                     prior_segments=(128,))
    print("sparse select at 8,192 candidates", flush=True)
    s = Session(wl, seed=121, layer=0, session=0)
    n_hist = 128 * 64
    assert n_hist == 8192 and wl.P == sa.SPARSE_KEY_BLOCK
    keep = sa.sparse_keep(n_hist, 25)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    got = sa.sparse_select(s.geom, it).cpu().numpy()
    want, scores = s.oracle_select(n_hist, keep)
    swaps = check_block_lists(got, want, scores, 1e-4)
    print(f"near-tie swaps {swaps}", flush=True)
    s.set_sparse(want, n_hist)
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    rows = si.sample_rows(wl.Lq, 64, 3, [255, 256, wl.Lq - 1])
    _check(s, "attention over 2,048 of 8,192 blocks", rows=rows)
    # one more candidate than the bound is refused
    it.n_hist_frames = n_hist + 1
    with pytest.raises(sa.SegAttnError):
        sa.sparse_select(s.geom, it)


def test_sparse_partial_history_and_single_block():
    """Candidates are the first 5 of 9 history frames (the other 4 stay
    dense); then a single kept block."""
    wl = si.Workload("partial", heads=2, lat_t=3, lat_h=8, lat_w=16, n_text=24,
                     prior_segments=(3,))
    s = Session(wl, seed=123, layer=0, session=0)
    for n_hist, keep in ((5, 3), (9, 1)):
        lists, _ = s.oracle_select(n_hist, keep)
        s.set_sparse(lists, n_hist)
        sa.segment_attention(s.geom, [s.item()])
        torch.cuda.synchronize()
        _check(s, f"{n_hist} candidate frames, keep {keep}")


def test_windows_at_the_table_bound():
    """Frames of 16 tokens and 3,616 text keys with seeded windows: the
    workgroup table holds 18 rows of 113 words."""
    wl = si.Workload("wmax", heads=2, lat_t=4, lat_h=4, lat_w=4, n_text=3616,
                     prior_segments=(2,))
    s = Session(wl, seed=125, layer=0, session=0)
    s.set_windows(si.text_windows(wl, 125, s.S * wl.lat_t, n_actions=9).numpy())
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(64), si.sample_rows(wl.Lq, 128, 5, [64, 255, 256])])
    rows = np.unique(rows)
    _check(s, "windows at the table bound", rows=rows)
