"""GPU parity of block-sparse history attention against the oracle.

The method: after the first denoising steps only a quarter of the candidate
video blocks are attended ("Hy-Nomas en una RTX 4090", "El preset de una
GPU"); oracle/sparse.py states the readings (64-token blocks of the history
frames, 256-row query blocks, pooled q . k scores, ceil(25 %) kept, ties to the
lower index).

Two halves, checked apart so that neither takes an input from the other:
- sparse_select (GPU) against the oracle's selection from the same seeded
  inputs. The kernel scores in fp32, the oracle in fp64, so a block may trade
  places with another only when their oracle scores lie within a small
  tolerance of the list's threshold; the lists must otherwise be equal, and
  are checked to be ascending, distinct and in range.
- segment_attention with block lists that the oracle selected, against the
  oracle's sparse attention with the same lists (bf16 and e4m3 bars as for
  the dense path), whole and split tiles, with timed windows, and a full list
  that is bitwise the dense result.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists, compare

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, REL_L2 = 2e-2, 2e-3, 1e-2
LSE_ATOL = 4e-3


def _wl(name, H, F, lh, lw, n_text, prior, kv):
    return si.Workload(name, heads=H, lat_t=F, lat_h=lh, lat_w=lw, n_text=n_text,
                       prior_segments=(prior,), kv_dtype=kv, scale_factors=(kv == "fp8"))


def _check(s, kv, label):
    got, got_lse = s.gpu_out()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse)), label
    if kv == "bf16":
        want, want_lse = s.oracle()
        _, _, rel = compare(got, want, MAX_ABS, MEAN_ABS, label)
        assert rel <= REL_L2, label
        np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0, err_msg=label)
    else:
        want, want_lse, bound = s.oracle_fp8_cache()
        err = np.abs(got - want)
        worst = float(np.max(err / (bound + 5e-3)))
        print(f"{label}: max_abs={err.max():.3e} max(err / (bound + 5e-3))={worst:.3f}", flush=True)
        assert worst <= 1.0, label
        np.testing.assert_allclose(got_lse, want_lse, atol=2e-2, rtol=0, err_msg=label)
    return got


CASES = [
    # name, H, F, lat_h, lat_w, n_text, prior segments, keep percent
    ("s_p128", 2, 4, 8, 16, 40, 3, 25),     # 12 history frames x 2 blocks = 24 candidates
    ("s_p80", 3, 3, 8, 10, 37, 4, 25),      # blocks of 64 and 16 keys; ragged text
    ("s_keep1", 2, 2, 8, 8, 16, 3, 1),      # a single kept block
    ("s_p24", 2, 4, 4, 6, 16, 3, 25),       # frames of 24 tokens (e4m3 planes of 32 slots)
]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_matches_oracle(case, kv):
    name, H, F, lh, lw, nt, prior, pct = case
    print(f"sparse select case={name} kv={kv}", flush=True)
    wl = _wl(name, H, F, lh, lw, nt, prior, kv)
    s = Session(wl, seed=91, layer=0, session=0)
    n_hist = prior * F
    n_cand = n_hist * -(-wl.P // 64)
    keep = sa.sparse_keep(n_cand, pct)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    got = sa.sparse_select(s.geom, it).cpu().numpy()
    torch.cuda.synchronize()
    want, scores = s.oracle_select(n_hist, keep)
    swaps = check_block_lists(got, want, scores, 1e-4 if kv == "bf16" else 1e-3)
    print(f"{name} {kv}: {n_cand} candidates, keep {keep}, near-tie swaps {swaps}", flush=True)
    # determinism: a second selection is bitwise the first
    again = sa.sparse_select(s.geom, it).cpu().numpy()
    assert np.array_equal(again, got)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_sparse_attention_matches_oracle(case, kv):
    name, H, F, lh, lw, nt, prior, pct = case
    print(f"sparse attention case={name} kv={kv}", flush=True)
    wl = _wl(name, H, F, lh, lw, nt, prior, kv)
    s = Session(wl, seed=93, layer=0, session=0)
    n_hist = prior * F
    keep = sa.sparse_keep(n_hist * -(-wl.P // 64), pct)
    lists, _ = s.oracle_select(n_hist, keep)
    s.set_sparse(lists, n_hist)
    sa.segment_attention(s.geom, [s.item()], workspace=None)
    torch.cuda.synchronize()
    got = _check(s, kv, f"{name} {kv} whole")
    # the sparsity matters: the dense answer is far from the sparse one
    if kv == "bf16":
        want, _ = s.oracle()
        lists_kept = s.block_lists
        s.clear_sparse()
        dense, _ = s.oracle()
        s.set_sparse(lists_kept, n_hist)
        assert np.linalg.norm(got - want) < 0.1 * np.linalg.norm(want - dense)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sparse_split_tiles(kv):
    """Split parts of a sparse work tile divide its logical tiles (kept blocks
    first); split and whole runs both meet the bar."""
    wl = _wl("s_split", 4, 8, 8, 16, 64, 3, kv)     # 12 kept + 16 own + 1 text tiles
    s = Session(wl, seed=95, layer=0, session=0)
    n_hist = 3 * 8
    keep = sa.sparse_keep(n_hist * 2, 25)
    lists, _ = s.oracle_select(n_hist, keep)
    s.set_sparse(lists, n_hist)
    assert sa.segment_attention_workspace(s.geom, [s.item()]) > 0
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check(s, kv, f"sparse split {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_full_list_is_bitwise_dense(kv):
    """Every candidate kept, in order: the sparse walk visits the dense key
    order, so the result is bitwise the dense one (whole and split tiles)."""
    wl = _wl("s_full", 2, 3, 8, 16, 24, 2, kv)
    s = Session(wl, seed=97, layer=0, session=0)
    for ws in (None, "auto"):
        s.clear_sparse()
        sa.segment_attention(s.geom, [s.item()], workspace=ws)
        torch.cuda.synchronize()
        dense, dense_lse = s.gpu_out()
        n_hist = 2 * 3
        n_cand = n_hist * 2
        nq = -(-wl.Lq // 256)
        s.set_sparse(np.tile(np.arange(n_cand, dtype=np.int32), (wl.heads, nq, 1)), n_hist)
        sa.segment_attention(s.geom, [s.item()], workspace=ws)
        torch.cuda.synchronize()
        got, got_lse = s.gpu_out()
        assert np.array_equal(got, dense) and np.array_equal(got_lse, dense_lse), ws


def test_sparse_with_windows():
    """Block-sparse history and timed text windows in one call."""
    wl = _wl("s_win", 2, 4, 8, 16, 40, 3, "bf16")
    s = Session(wl, seed=99, layer=0, session=0)
    n_hist = 12
    lists, _ = s.oracle_select(n_hist, sa.sparse_keep(24, 25))
    s.set_sparse(lists, n_hist)
    s.set_windows(si.text_windows(wl, 99, s.S * wl.lat_t).numpy())
    sa.segment_attention(s.geom, [s.item()])
    torch.cuda.synchronize()
    _check(s, "bf16", "sparse + windows")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_select_then_attend(kv):
    """The whole sparse pass on the GPU: lists from sparse_select, then the
    attention. Query blocks whose GPU list equals the oracle's (all of them
    unless a near-tie swapped a block) are compared with the oracle's sparse
    attention over its own lists."""
    wl = _wl("s_e2e", 2, 4, 8, 16, 40, 3, kv)
    s = Session(wl, seed=101, layer=0, session=0)
    n_hist = 12
    keep = sa.sparse_keep(24, 25)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    d_lists = sa.sparse_select(s.geom, it)
    it.block_list = d_lists
    sa.segment_attention(s.geom, [it])
    torch.cuda.synchronize()
    got_lists = d_lists.cpu().numpy()
    want_lists, scores = s.oracle_select(n_hist, keep)
    check_block_lists(got_lists, want_lists, scores, 1e-4 if kv == "bf16" else 1e-3)
    s.set_sparse(want_lists, n_hist)
    same = np.all(got_lists == want_lists, axis=(0, 2))        # per query block, all heads
    rows = np.concatenate([np.arange(i * 256, min(wl.Lq, i * 256 + 256))
                           for i in range(len(same)) if same[i]])
    assert len(rows) > 0
    got, got_lse = s.gpu_out(rows=rows)
    if kv == "bf16":
        want, want_lse = s.oracle(rows=rows)
        compare(got, want, MAX_ABS, MEAN_ABS, "select then attend")
        np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0)
    else:
        want, want_lse, bound = s.oracle_fp8_cache(rows=rows)
        assert np.all(np.abs(got - want) <= bound + 5e-3)
        np.testing.assert_allclose(got_lse, want_lse, atol=2e-2, rtol=0)
