"""Camera cross-attention with a block-diagonal frame mask (oracle, test-only).

Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
(ai.thesatyajit.com), section "The camera": after each block a small
cross-attention module lets the video tokens read camera tokens, one per
latent frame (four consecutive 4x4 camera-to-world matrices flattened into a
64-wide vector, matching the VAE's 4x time compression); with a camera chunk
size of 1 the mask is block-diagonal, so latent frame t attends only to its
own camera token. The same page gives the camera key/value projection as
2,048 x 128: one 128-wide key/value head.

Readings taken here: the video queries of latent frame t (rows t*P ..
t*P + P - 1 of the segment, raster order) see the camera tokens of chunk
floor(t / c), i.e. tokens c*floor(t/c) .. c*floor(t/c) + c - 1 (those that
exist); no rotary embedding; softmax scale 1/sqrt(128) unless given; the
camera keys and values have either one head shared by every query head (the
2,048 x 128 projection) or one head per query head.

Everything here is plain numpy in fp64.
"""

import numpy as np

from .attention import attention


def camera_visibility(n_frames, P, n_cam, chunk):
    """bool [n_frames * P, n_cam]: camera tokens each video query row sees."""
    t = np.arange(n_frames * P) // P
    lo = (t // chunk) * chunk
    j = np.arange(n_cam)
    return (j[None, :] >= lo[:, None]) & (j[None, :] < lo[:, None] + chunk)


def camera_attention(q, cam_k, cam_v, P, chunk, scale=None):
    """q [n_frames * P, H, D] video queries; cam_k, cam_v [n_cam, Hk, D] with
    Hk = 1 (shared) or H. Returns (out [rows, H, D], lse [rows, H])."""
    q = np.asarray(q, dtype=np.float64)
    cam_k = np.asarray(cam_k, dtype=np.float64)
    cam_v = np.asarray(cam_v, dtype=np.float64)
    rows, H, D = q.shape
    n_frames = rows // P
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    vis = camera_visibility(n_frames, P, cam_k.shape[0], chunk)
    out = np.zeros(q.shape)
    lse = np.zeros((rows, H))
    for h in range(H):
        hk = 0 if cam_k.shape[1] == 1 else h
        out[:, h], lse[:, h] = attention(q[:, h], cam_k[:, hk], cam_v[:, hk], scale, vis)
    return out, lse
