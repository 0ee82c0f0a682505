"""Pins for oracle.attention (dense softmax attention in fp64).

Checked against: closed forms (uniform V gives V, a single key copies its
value, Q = 0 gives the mean of V, one dominant key gives its value), key
permutation invariance, the split/merge identity of log-sum-exp partials,
scalar brute-force triple loops written independently here, torch's
scaled_dot_product_attention in float64 on the CPU (an independent library
routine for the same definition) and scipy's logsumexp for the LSE. Timed
text windows: masked attention equals deleting the invisible keys, the
visibility cases of the reading, torch's SDPA with a boolean mask.
"""

import math

import numpy as np
import torch
from scipy.special import logsumexp

from oracle import attention, rope


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_v_gives_v():
    q, k = _rand((9, 128), 0), _rand((40, 128), 1)
    v = np.tile(_rand((1, 128), 2), (40, 1))
    o, _ = attention.attention(q, k, v, 1 / math.sqrt(128))
    np.testing.assert_allclose(o, np.tile(v[:1], (9, 1)), rtol=0, atol=1e-14)


def test_single_key_copies_value():
    q, k, v = _rand((5, 128), 3), _rand((1, 128), 4), _rand((1, 128), 5)
    o, lse = attention.attention(q, k, v, 0.1)
    assert np.array_equal(o, np.tile(v, (5, 1)))
    np.testing.assert_allclose(lse, 0.1 * (q @ k[0]), rtol=1e-14)


def test_zero_query_gives_mean_and_counts_keys():
    n = 77
    k = _rand((n, 128), 6)
    v = np.zeros((n, 128))
    v[np.arange(n), np.arange(n) % 128] = 1.0      # one-hot column per key
    o, lse = attention.attention(np.zeros((3, 128)), k, v, 0.088)
    counts = np.bincount(np.arange(n) % 128, minlength=128) / n
    np.testing.assert_allclose(o, np.tile(counts, (3, 1)), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-14)


def test_dominant_key():
    k = _rand((50, 128), 7) * 0.01
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    k[17, 0] = 1000.0
    v = _rand((50, 128), 8)
    o, _ = attention.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o[0], v[17], rtol=0, atol=1e-12)


def test_key_permutation_invariance():
    q, k, v = _rand((6, 128), 9), _rand((60, 128), 10), _rand((60, 128), 11)
    perm = np.random.default_rng(12).permutation(60)
    o1, l1 = attention.attention(q, k, v, 0.09)
    o2, l2 = attention.attention(q, k[perm], v[perm], 0.09)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_split_merge_identity():
    q, k, v = _rand((6, 128), 13), _rand((70, 128), 14), _rand((70, 128), 15)
    o, l = attention.attention(q, k, v, 0.1)
    oa, la = attention.attention(q, k[:23], v[:23], 0.1)
    ob, lb = attention.attention(q, k[23:], v[23:], 0.1)
    om, lm = attention.merge_partials(oa, la, ob, lb)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, l, rtol=1e-13)


def test_brute_force_triple_loop():
    M, N, D = 4, 11, 128
    q, k, v = _rand((M, D), 16), _rand((N, D), 17), _rand((N, D), 18)
    scale = 1 / math.sqrt(D)
    o, lse = attention.attention(q, k, v, scale)
    for i in range(M):
        s = [scale * sum(q[i, c] * k[j, c] for c in range(D)) for j in range(N)]
        z = sum(math.exp(x) for x in s)
        assert abs(lse[i] - math.log(z)) < 1e-12
        for c in range(D):
            ref = sum(math.exp(s[j]) * v[j, c] for j in range(N)) / z
            assert abs(o[i, c] - ref) < 1e-13


def test_matches_torch_sdpa_fp64():
    q, k, v = _rand((33, 128), 19), _rand((150, 128), 20), _rand((150, 128), 21)
    o, lse = attention.attention(q, k, v, 1 / math.sqrt(128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, logsumexp((q @ k.T) / math.sqrt(128), axis=1), rtol=1e-13)


def test_large_logits_stable():
    q = _rand((4, 128), 22) * 40
    k = _rand((30, 128), 23) * 40
    v = _rand((30, 128), 24)
    o, lse = attention.attention(q, k, v, 1 / math.sqrt(128))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_segment_attention_rotates_then_attends():
    """segment_attention == rotate Q and K by their positions, then attention per head."""
    H, D = 2, 128
    Lq, Lk = 20, 45
    q, k, v = _rand((Lq, H, D), 25), _rand((Lk, H, D), 26), _rand((Lk, H, D), 27)
    qp = np.random.default_rng(28).integers(0, 30, (Lq, 3))
    kp = np.random.default_rng(29).integers(0, 30, (Lk, 3))
    o, lse = attention.segment_attention(q, qp, k, kp, v, theta=256.0)
    qr, kr = rope.rope3d(q, qp, theta=256.0), rope.rope3d(k, kp, theta=256.0)
    for h in range(H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qr[:, h])[None], torch.from_numpy(kr[:, h])[None],
            torch.from_numpy(v[:, h])[None])[0].numpy()
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-12, atol=1e-13)
    rows = [0, 7, 19]
    o2, l2 = attention.segment_attention(q, qp, k, kp, v, theta=256.0, rows=rows, chunk=2)
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l2, lse[rows], rtol=1e-13)


def test_empty_key_set_rejected():
    try:
        attention.attention(np.zeros((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    except ValueError:
        return
    raise AssertionError("expected ValueError")


# ---- timed text windows ------------------------------------------------------------
def _window_case(seed):
    """A small session: 3 video frames of 4 query rows, 3 text query rows; keys
    are 10 video keys and 6 text keys with assorted windows (all frames, one
    frame, an empty range, a range past the segment)."""
    rng = np.random.default_rng(seed)
    q_frame = np.array([5] * 4 + [6] * 4 + [7] * 4 + [-1] * 3)
    key_text = np.array([-1] * 10 + list(range(6)))
    window = np.array([[0, 1 << 30], [6, 6], [7, 5], [5, 6], [8, 9], [7, 7]])
    q = rng.standard_normal((len(q_frame), 32))
    k = rng.standard_normal((len(key_text), 32))
    v = rng.standard_normal((len(key_text), 32))
    return q_frame, key_text, window, q, k, v


def test_text_window_is_deletion_of_invisible_keys():
    """Masked attention of each row equals plain attention over the keys that
    row keeps, computed by deleting the others from the key set."""
    q_frame, key_text, window, q, k, v = _window_case(41)
    vis = attention.timed_text_visibility(q_frame, key_text, window)
    out, lse = attention.attention(q, k, v, 0.2, vis)
    for r in range(len(q_frame)):
        keep = np.flatnonzero(vis[r])
        o1, l1 = attention.attention(q[r:r + 1], k[keep], v[keep], 0.2)
        np.testing.assert_allclose(out[r], o1[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[r], l1[0], rtol=1e-13)


def test_text_window_visibility_cases():
    """Text rows and video keys are never masked; an all-frames window masks
    nothing; the one-frame window [6, 6] reaches frame 6 only; the empty range
    [7, 5] reaches no video row; a window past the segment reaches none."""
    q_frame, key_text, window, _, _, _ = _window_case(42)
    vis = attention.timed_text_visibility(q_frame, key_text, window)
    assert vis[:, :10].all()                         # video keys
    assert vis[12:, :].all()                         # text rows
    assert vis[:12, 10].all()                        # window (0, 2^30)
    assert np.array_equal(vis[:12, 11], q_frame[:12] == 6)
    assert not vis[:12, 12].any()                    # (7, 5): empty
    assert np.array_equal(vis[:12, 13], q_frame[:12] <= 6)
    assert not vis[:12, 14].any()                    # (8, 9): past the segment
    assert np.array_equal(vis[:12, 15], q_frame[:12] == 7)


def test_text_window_matches_torch_masked_sdpa():
    """Against torch's scaled_dot_product_attention with a boolean mask, fp64."""
    q_frame, key_text, window, q, k, v = _window_case(43)
    vis = attention.timed_text_visibility(q_frame, key_text, window)
    out, _ = attention.attention(q, k, v, 1.0 / math.sqrt(32), vis)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(vis)[None])[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_segment_attention_with_windows_all_frames_is_unmasked():
    """Windows that cover every frame leave segment_attention unchanged."""
    H, D = 2, 128
    Lq, Lk, nt = 12, 30, 5
    q, k, v = _rand((Lq, H, D), 44), _rand((Lk, H, D), 45), _rand((Lk, H, D), 46)
    qp = np.random.default_rng(47).integers(0, 30, (Lq, 3))
    kp = np.random.default_rng(48).integers(0, 30, (Lk, 3))
    q_frame = np.array([3] * 8 + [-1] * 4)
    key_text = np.array([-1] * (Lk - nt) + list(range(nt)))
    win = np.array([[0, 100]] * nt)
    o, l = attention.segment_attention(q, qp, k, kp, v, q_frame=q_frame, key_text=key_text,
                                       text_window=win)
    o0, l0 = attention.segment_attention(q, qp, k, kp, v)
    np.testing.assert_allclose(o, o0, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l, l0, rtol=1e-13)


def test_row_that_sees_no_key_rejected():
    try:
        attention.attention(np.zeros((1, 4)), np.zeros((2, 4)), np.zeros((2, 4)), 1.0,
                            np.zeros((1, 2), dtype=bool))
    except ValueError:
        return
    raise AssertionError("expected ValueError")
