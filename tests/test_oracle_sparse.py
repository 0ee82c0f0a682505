"""Pins of the block-sparse history oracle (oracle/sparse.py) against things
other than itself: brute-force loops on tiny inputs, a planted dominant block,
ties, the dense limit, and deletion of the hidden blocks from the key set."""

import math

import numpy as np
import pytest

from oracle import attention, sparse


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_keep_count():
    assert sparse.keep_count(420, 25) == 105
    assert sparse.keep_count(3360, 25) == 840
    assert sparse.keep_count(3, 25) == 1          # ceil(0.75)
    assert sparse.keep_count(5, 25) == 2          # ceil(1.25)
    assert sparse.keep_count(1, 25) == 1
    assert sparse.keep_count(0, 25) == 0
    assert sparse.keep_count(7, 100) == 7
    assert sparse.keep_count(7, 0) == 1           # at least one block


def test_candidate_blocks_of_a_ragged_frame():
    # P = 136: blocks of 64, 64 and 8 tokens per frame
    b = sparse.candidate_blocks(2, 136)
    assert b == [(0, 0, 64), (0, 64, 64), (0, 128, 8), (1, 0, 64), (1, 64, 64), (1, 128, 8)]
    assert sparse.candidate_blocks(0, 136) == []


def test_selection_matches_brute_force_loops():
    """Pooling, scoring, ordering and the ascending list, written as loops."""
    H, D, P, nf = 2, 6, 10, 3                 # blocks of 4 keys: 3 per frame (4, 4, 2)
    Lq, bq, bk, keep = 7, 3, 4, 4
    q = _rand((Lq, H, D), 1)
    k = _rand((nf * P, H, D), 2)
    got = sparse.select_blocks(q, k, nf, P, keep, block=bk, block_q=bq)
    per = 3
    for h in range(H):
        for qb in range(3):
            rows = range(qb * bq, min(Lq, qb * bq + bq))
            pq = [sum(q[r, h, d] for r in rows) / len(rows) for d in range(D)]
            scores = []
            for f in range(nf):
                for j in range(per):
                    toks = range(f * P + j * bk, f * P + min(P, j * bk + bk))
                    pk = [sum(k[t, h, d] for t in toks) / len(toks) for d in range(D)]
                    scores.append(sum(pq[d] * pk[d] for d in range(D)))
            ranked = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
            assert list(got[h, qb]) == sorted(ranked[:keep])


def test_planted_block_is_kept():
    """A block whose keys all point along the query block's mean is the only one kept at keep = 1."""
    H, D, P, nf = 1, 8, 64, 4
    q = _rand((40, H, D), 3)
    k = _rand((nf * P, H, D), 4) * 0.1
    qm = q[:, 0].mean(axis=0)
    k[2 * P + 0:2 * P + 64, 0] = 5.0 * qm / np.linalg.norm(qm)     # frame 2, block 0
    got = sparse.select_blocks(q, k, nf, P, 1)
    assert got.shape == (1, 1, 1) and got[0, 0, 0] == 2


def test_ties_go_to_the_lower_block():
    """Identical blocks score the same: the lower index is kept."""
    H, D, P, nf = 1, 4, 64, 3
    q = _rand((10, H, D), 5)
    base = _rand((P, H, D), 6)
    k = np.concatenate([base * 0.5, base, base])   # frames 1 and 2 identical
    qm = q[:, 0].mean(axis=0)
    if float(qm @ base[:, 0].mean(axis=0)) < 0:    # make the duplicates the best blocks
        k = -k
        k[:P] = -k[:P]
    got = sparse.select_blocks(q, k, nf, P, 1)
    assert got[0, 0, 0] == 1


def test_sparse_attention_with_every_block_is_dense():
    H, D, P, nf = 2, 16, 64, 3
    Lq, own = 30, 2 * P
    q = _rand((Lq, H, D), 7)
    k = _rand((nf * P + own, H, D), 8)
    v = _rand((nf * P + own, H, D), 9)
    pos = np.zeros((Lq, 3))
    kpos = np.zeros((k.shape[0], 3))
    lists = np.tile(np.arange(nf)[None, None, :], (H, 1, 1)).astype(np.int32)
    dense, dl = attention.segment_attention(q, pos, k, kpos, v, split=(4, 6, 6), theta=256.0)
    sp, sl = attention.segment_attention(q, pos, k, kpos, v, split=(4, 6, 6), theta=256.0,
                                         block_lists=lists, n_hist_frames=nf, P=P)
    assert np.array_equal(dense, sp) and np.array_equal(dl, sl)


def test_sparse_attention_is_deletion_of_unkept_blocks():
    """Per head and query block: attention with the unkept candidate blocks
    hidden equals attention over the key set with those blocks deleted."""
    H, D, P, nf = 2, 16, 80, 3          # blocks of 64 and 16 keys per frame
    Lq, own = 300, 2 * P                # two query blocks (256 + 44 rows)
    q = _rand((Lq, H, D), 10)
    k = _rand((nf * P + own, H, D), 11)
    v = _rand((nf * P + own, H, D), 12)
    pos = np.zeros((Lq, 3))
    kpos = np.zeros((k.shape[0], 3))
    keep = 2
    lists = sparse.select_blocks(q, k[:nf * P], nf, P, keep)
    assert lists.shape == (H, 2, keep)
    out, lse = attention.segment_attention(q, pos, k, kpos, v, split=(4, 6, 6), theta=256.0,
                                           block_lists=lists, n_hist_frames=nf, P=P)
    blocks = sparse.candidate_blocks(nf, P)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        for qb, rows in enumerate((range(0, 256), range(256, 300))):
            keys = [f * P + s + t for b in lists[h, qb] for (f, s, n) in [blocks[b]] for t in range(n)]
            keys += list(range(nf * P, k.shape[0]))
            o, l = attention.attention(q[list(rows), h], k[keys, h], v[keys, h], scale)
            np.testing.assert_allclose(out[list(rows), h], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[list(rows), h], l, rtol=1e-12, atol=1e-12)


def test_sparse_and_windows_combine():
    """Both masks at once: a row keeps a key only if both keep it."""
    H, D, P, nf = 1, 8, 64, 2
    Lq, nt = 20, 6
    q = _rand((Lq, H, D), 13)
    k = _rand((nf * P + P + nt, H, D), 14)
    v = _rand((nf * P + P + nt, H, D), 15)
    pos = np.zeros((Lq, 3))
    kpos = np.zeros((k.shape[0], 3))
    lists = np.array([[[1]]], dtype=np.int32)
    q_frame = np.array([5] * 10 + [6] * 4 + [-1] * 6)
    key_text = np.concatenate([-np.ones(nf * P + P, dtype=np.int64), np.arange(nt)])
    win = np.array([[5, 5], [6, 6], [0, 9], [7, 8], [5, 6], [6, 5]])
    out, _ = attention.segment_attention(q, pos, k, kpos, v, split=(2, 2, 4), theta=256.0,
                                         q_frame=q_frame, key_text=key_text, text_window=win,
                                         block_lists=lists, n_hist_frames=nf, P=P)
    vis = (sparse.sparse_visibility(np.arange(Lq), lists[0], nf, P, k.shape[0])
           & attention.timed_text_visibility(q_frame, key_text, win))
    assert not vis[:, :P].any() and vis[:, P:2 * P].all()
    want, _ = attention.attention(q[:, 0], k[:, 0], v[:, 0], 1.0 / math.sqrt(D), vis)
    np.testing.assert_allclose(out[:, 0], want, rtol=1e-13, atol=1e-13)
