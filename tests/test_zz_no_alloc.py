"""sparse_select_noalloc (pooled keys in the library's static device scratch)
against sparse_select (pooled keys in a caller workspace), through the C ABI.

Both run the same kernels, so the block lists must be equal bit for bit. Two
calls in a row on one GPU, the second on a smaller input (fewer heads and
candidates, another cache dtype), so the second reads a scratch that still
holds the first call's pooled keys; then the first input once more. The
small input's lists are also checked against the oracle's selection (up to
near-ties at the threshold, as for sparse_select). The refusal of inputs
beyond the scratch is checked on the host (tests/test_abi_cpu.py).
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists

pytestmark = pytest.mark.gpu


def _lists(s, n_hist, percent):
    it = s.item()
    keep = sa.sparse_keep(n_hist * -(-s.wl.P // sa.SPARSE_KEY_BLOCK), percent)
    it.n_hist_frames, it.keep_blocks = n_hist, keep
    want = sa.sparse_select(s.geom, it)
    got = torch.full_like(want, -7)
    sa.sparse_select_noalloc(s.geom, it, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy(), keep


def test_noalloc_select_matches_workspace_select_twice():
    # 16 heads, 880-token frames (14 key blocks each), 24 history frames:
    # 336 candidates, 16 x 336 x 512 B = 2.6 MiB of pooled keys; 3,776 query
    # rows in 15 query blocks.
    big = si.Workload("noalloc_big", heads=16, lat_t=4, lat_h=22, lat_w=40, n_text=256,
                      prior_segments=(6,))
    # 2 heads, 128-token frames (2 blocks each), e4m3 cache, 12 history frames.
    small = si.Workload("noalloc_small", heads=2, lat_t=4, lat_h=8, lat_w=16, n_text=40,
                        prior_segments=(3,), kv_dtype="fp8", scale_factors=True)
    print("noalloc: 16 heads, 336 candidates (bf16)", flush=True)
    sb = Session(big, seed=131, layer=0, session=0)
    got, want, keep = _lists(sb, 24, 25)
    assert want.shape == (16, 15, keep) and keep == 84
    np.testing.assert_array_equal(got, want)

    print("noalloc: 2 heads, 24 candidates (e4m3), after the larger call", flush=True)
    ss = Session(small, seed=132, layer=0, session=0)
    got2, want2, keep2 = _lists(ss, 12, 25)
    assert want2.shape == (2, 3, keep2) and keep2 == 6
    np.testing.assert_array_equal(got2, want2)
    lists, scores = ss.oracle_select(12, keep2)
    check_block_lists(got2, lists, scores, 1e-4)

    print("noalloc: the first input again", flush=True)
    got3, _, _ = _lists(sb, 24, 25)
    np.testing.assert_array_equal(got3, want)


def test_noalloc_select_on_a_side_stream():
    """The call is stream-ordered: on a side stream, after the block list was
    filled on that stream, it matches the workspace call."""
    wl = si.Workload("noalloc_stream", heads=4, lat_t=3, lat_h=8, lat_w=16, n_text=24,
                     prior_segments=(4,), kv_dtype="int8")
    print("noalloc: 4 heads, int8 cache, side stream", flush=True)
    s = Session(wl, seed=133, layer=0, session=0)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = 12, 5
    want = sa.sparse_select(s.geom, it)
    side = torch.cuda.Stream()
    got = torch.empty_like(want)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got.fill_(-1)
        sa.sparse_select_noalloc(s.geom, it, got, stream=side)
    side.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), want.cpu().numpy())


def test_noalloc_select_fills_the_whole_scratch():
    """16 heads x 4,096 candidates (4,096 history frames of 64 tokens, one
    block each) x 512 bytes: exactly the 32 MiB scratch. The lists equal the
    workspace call's bit for bit; one candidate more is refused."""
    wl = si.Workload("noalloc_max", heads=16, lat_t=64, lat_h=8, lat_w=8, n_text=16,
                     prior_segments=(64,))
    print("noalloc: 16 heads x 4,096 candidates, the whole scratch", flush=True)
    s = Session(wl, seed=134, layer=0, session=0)
    n_hist = 64 * 64
    assert 16 * n_hist * 512 == sa.SPARSE_SCRATCH_BYTES
    got, want, keep = _lists(s, n_hist, 25)
    assert keep == 1024
    np.testing.assert_array_equal(got, want)
    it = s.item()
    it.n_hist_frames, it.keep_blocks = n_hist + 1, keep
    lists = torch.empty((16, -(-wl.Lq // sa.SPARSE_QUERY_BLOCK), keep), dtype=torch.int32,
                        device="cuda")
    with pytest.raises(sa.SegAttnError) as e:
        sa.sparse_select_noalloc(s.geom, it, lists)
    assert e.value.status == 6 and "static scratch" in str(e.value)
