"""Pins of the camera cross-attention oracle (oracle/camera.py): the
block-diagonal case copies each frame's camera value, a chunk spanning every
frame is plain attention, the mask matches a brute-force loop, and each
frame's rows equal attention over its chunk's tokens alone."""

import math

import numpy as np

from oracle import attention, camera


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_visibility_brute_force():
    n_frames, P, n_cam = 7, 3, 8
    for chunk in (1, 2, 3, 8):
        vis = camera.camera_visibility(n_frames, P, n_cam, chunk)
        for r in range(n_frames * P):
            t = r // P
            for j in range(n_cam):
                assert vis[r, j] == (j // chunk == t // chunk)


def test_chunk_one_copies_the_frames_camera_value():
    """One key per row: softmax weight 1, the output is that value exactly."""
    n_frames, P, H, D = 5, 4, 3, 8
    q = _rand((n_frames * P, H, D), 1)
    ck = _rand((n_frames, 1, D), 2)
    cv = _rand((n_frames, 1, D), 3)
    out, lse = camera.camera_attention(q, ck, cv, P, 1)
    for r in range(n_frames * P):
        t = r // P
        for h in range(H):
            assert np.array_equal(out[r, h], cv[t, 0])
            np.testing.assert_allclose(lse[r, h], q[r, h] @ ck[t, 0] / math.sqrt(D), rtol=1e-14)


def test_one_chunk_is_plain_attention():
    n_frames, P, H, D = 3, 5, 2, 16
    q = _rand((n_frames * P, H, D), 4)
    ck = _rand((n_frames, H, D), 5)
    cv = _rand((n_frames, H, D), 6)
    out, lse = camera.camera_attention(q, ck, cv, P, n_frames)
    for h in range(H):
        o, l = attention.attention(q[:, h], ck[:, h], cv[:, h], 1.0 / math.sqrt(D))
        np.testing.assert_allclose(out[:, h], o, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lse[:, h], l, rtol=1e-14, atol=1e-14)


def test_each_frame_attends_its_chunk_alone():
    """Chunk 2 over 5 frames (chunks {0,1}, {2,3}, {4}), shared and per-head
    keys: every frame's rows equal attention over its chunk's tokens."""
    n_frames, P, H, D = 5, 3, 2, 8
    q = _rand((n_frames * P, H, D), 7)
    for hk in (1, H):
        ck = _rand((n_frames, hk, D), 8 + hk)
        cv = _rand((n_frames, hk, D), 9 + hk)
        out, _ = camera.camera_attention(q, ck, cv, P, 2)
        for t in range(n_frames):
            keys = [j for j in range(n_frames) if j // 2 == t // 2]
            rows = slice(t * P, (t + 1) * P)
            for h in range(H):
                kh = 0 if hk == 1 else h
                o, _ = attention.attention(q[rows, h], ck[keys, kh], cv[keys, kh], 1.0 / math.sqrt(D))
                np.testing.assert_allclose(out[rows, h], o, rtol=1e-13, atol=1e-13)
