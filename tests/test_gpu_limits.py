"""GPU parity at the limits the C ABI states, against the oracle.

- sparse_select at SA_MAX_SPARSE_CANDIDATES (8,192 candidate blocks: 8,192
  history frames of 64 tokens), the selection kernel's largest radix-select
  and scan, and the attention over its lists;
- block-sparse history whose candidates are only part of the history (the
  other history frames stay dense), and a single kept block;
- timed text windows at the window-table bound: frames of 16 tokens with
  3,616 text keys fill (255 / 16 + 3) * ceil(3616 / 32) = 2,034 of the 2,048
  table words (one more word is refused on the host: tests/test_abi_cpu.py);
- a key set of SA_MAX_FRAMES_KV frames (65,536 frames of 8 tokens, the
  history in a seeded random order), bf16 and e4m3, whole and split: one key
  tile per frame, so the key walk enters a new frame on every tile.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists, compare, prob_rounding_bound
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import rope as orope

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


def _fp8_stored(s):
    """The e4m3 cache's K and V of the session's key set, [Lk, H, D] float64,
    from the oracle's own append of each segment (quantise, then decode times
    the plane scale), taken in key-set order."""
    wl = s.wl
    F, H, D = wl.lat_t, wl.heads, wl.head_dim
    raw = [(seg, s.raw_k[seg].float().cpu().double().numpy(),
            s.raw_v[seg].float().cpu().double().numpy()) for seg in range(s.S + 1)]

    def one_segment(args):   # segments are independent: one per worker thread
        seg, kin, vin = args
        kc, ksc, vc, vsc = ocache.append_fp8(kin, vin, seg * F, wl.lat_h, wl.lat_w, wl.split,
                                             s.geom.rope_theta)
        return (ocache.dequant(kc, ksc[:, :, None, None]).transpose(0, 2, 1, 3),   # [F, P, H, D]
                ocache.dequant(vc, vsc[:, :, None, None]).transpose(0, 3, 1, 2))

    import concurrent.futures
    with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
        per_seg = list(ex.map(one_segment, raw))
    del raw
    fr = np.asarray(s.frames)
    k = np.concatenate([x[0] for x in per_seg])[fr].reshape(-1, H, D)
    v = np.concatenate([x[1] for x in per_seg])[fr].reshape(-1, H, D)
    del per_seg
    tk = s.text_k.float().cpu().double().numpy()
    tv = s.text_v.float().cpu().double().numpy()
    kc, ksc, vc, vsc = ocache.append_text_fp8(tk, tv)
    k = np.concatenate([k, ocache.dequant(kc, ksc[:, None, None]).transpose(1, 0, 2)])
    v = np.concatenate([v, ocache.dequant(vc, vsc[:, None, None]).transpose(2, 0, 1)])
    return k, v


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_key_set_at_the_frame_bound(kv):
    """65,536 frames in the key set (31 prior segments of 2,048 frames of
    2 x 4 tokens, history shuffled, and the segment's own 2,048 frames), one
    head, 16 text keys; sampled rows against the oracle, with the tiles run
    whole and split."""
    wl = si.Workload("maxframes", heads=1, lat_t=2048, lat_h=2, lat_w=4, n_text=16,
                     prior_segments=(31,), kv_dtype=kv, scale_factors=(kv == "fp8"))
    g = np.random.default_rng(si.derive_seed(127, "frame bound history"))
    history = [int(f) for f in g.permutation(31 * 2048)]
    print(f"{kv}: {len(history) + wl.lat_t} frames of {wl.P} tokens, one head", flush=True)
    s = Session(wl, seed=127, layer=0, session=0, history=history)
    assert len(s.frames) == sa.MAX_FRAMES_KV
    rows = si.sample_rows(wl.Lq, 48, 7, [255, 256, wl.Lq - 17, wl.Lq - 16])
    if kv == "bf16":
        want, want_lse = s.oracle(rows=rows)
    else:
        k, v = _fp8_stored(s)
        q = s.q.float().cpu().double().numpy()[rows]
        qr = orope.rope3d(q, s.q_positions()[rows], wl.split, s.geom.rope_theta)
        scale = 1.0 / np.sqrt(wl.head_dim)
        want, want_lse = oatt.attention(qr[:, 0], k[:, 0], v[:, 0], scale, None)
        sc = (qr[:, 0] @ k[:, 0].T) * scale
        p = np.exp(sc - sc.max(axis=1, keepdims=True))
        bound = prob_rounding_bound(p, np.abs(v[:, 0]))
        del k, v, sc, p
    for split in (False, True):
        label = f"{kv} at {sa.MAX_FRAMES_KV} frames, {'split' if split else 'whole'} tiles"
        print(label, flush=True)
        sa.segment_attention(s.geom, [s.item()], workspace="auto" if split else None)
        torch.cuda.synchronize()
        got, got_lse = s.gpu_out(rows=rows)
        if kv == "bf16":
            _, _, rel = compare(got, want, MAX_ABS, MEAN_ABS, label)
            assert rel <= REL_L2, label
            np.testing.assert_allclose(got_lse, want_lse, atol=LSE_ATOL, rtol=0, err_msg=label)
        else:
            err = np.abs(got[:, 0] - want)
            worst = float(np.max(err / (bound + 5e-3)))
            rel = float(np.linalg.norm(got[:, 0] - want) / np.linalg.norm(want))
            print(f"  max_abs={err.max():.3e} rel_l2={rel:.3e} max(err / (bound + 5e-3))={worst:.3f}",
                  flush=True)
            assert worst <= 1.0 and rel <= 0.05, label
            np.testing.assert_allclose(got_lse[:, 0], want_lse, atol=2e-2, rtol=0, err_msg=label)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_full_list_past_the_staged_kept_tiles(kv):
    """8,192 candidate tiles (128 prior segments of 64 one-tile frames), all
    kept in order: the sparse walk visits the dense key order, so the result
    is bitwise the dense one, whole and split. The e4m3 kernel stages at most
    4,096 kept tiles of a work tile in LDS and walks the rest from the list."""
    wl = si.Workload("fullkeep", heads=1, lat_t=64, lat_h=8, lat_w=8, n_text=16,
                     prior_segments=(128,), kv_dtype=kv, scale_factors=(kv == "fp8"))
    s = Session(wl, seed=129, layer=0, session=0)
    n_hist = 128 * 64
    nq = -(-wl.Lq // sa.SPARSE_QUERY_BLOCK)
    lists = np.tile(np.arange(n_hist, dtype=np.int32), (wl.heads, nq, 1))
    for ws in (None, "auto"):
        print(f"{kv}: keep all {n_hist} candidates, {'split' if ws else 'whole'} tiles", flush=True)
        s.clear_sparse()
        sa.segment_attention(s.geom, [s.item()], workspace=ws)
        torch.cuda.synchronize()
        dense, dense_lse = s.gpu_out()
        s.set_sparse(lists, n_hist)
        sa.segment_attention(s.geom, [s.item()], workspace=ws)
        torch.cuda.synchronize()
        got, got_lse = s.gpu_out()
        assert np.array_equal(got, dense) and np.array_equal(got_lse, dense_lse), ws
