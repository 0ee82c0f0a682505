"""3D rotary position embedding over (t, h, w) (oracle, test-only).

Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
(ai.thesatyajit.com), section "How one segment is made": each head of 128
dimensions is split [16, 56, 56] across the time, height and width axes, with
theta 256; the video token grid is 22 x 40 per latent frame with patch size
1x1x1.

Readings where the page is silent (each one also listed in the design notes):

* pairing: dimensions (2j, 2j+1) of an axis band form one rotation pair, as in
  the original rotary embedding (Su et al., RoFormer);
* frequencies: each band is an independent 1-D rotary embedding of size n,
  frequency of pair j = theta ** (-2j / n);
* positions: t is the absolute latent-frame index since the world started,
  (h, w) the row and column of the token in its frame; text tokens sit at
  (0, 0, 0), which is the identity rotation;
* only queries and keys are rotated, never values.
"""

import numpy as np


def axis_frequencies(n, theta):
    """Frequencies theta**(-2j/n) for j = 0 .. n/2-1 of one axis band (float64)."""
    if n % 2:
        raise ValueError("an axis band must have an even number of dims")
    j = np.arange(n // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / n)


def rope3d(x, pos, split=(16, 56, 56), theta=10000.0):
    """Rotate the last axis of ``x`` by the 3D rotary embedding at ``pos``.

    x:   float64 array [..., n_tokens, (heads,) dims] -- any shape whose
         second-to-last or third-to-last axis is the token axis matching pos.
         Supported shapes: [n, D] and [n, H, D].
    pos: int array [n, 3] of (t, h, w) per token.
    Returns a new float64 array of the same shape.
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    D = x.shape[-1]
    if sum(split) != D:
        raise ValueError("rope split must sum to the head dim")
    if x.ndim == 2:
        y = _rotate(x[:, None, :], pos, split, theta)[:, 0, :]
    elif x.ndim == 3:
        y = _rotate(x, pos, split, theta)
    else:
        raise ValueError("x must be [n, D] or [n, H, D]")
    return y


def _rotate(x, pos, split, theta):
    out = x.copy()
    off = 0
    for axis, n in enumerate(split):
        w = axis_frequencies(n, theta)                       # [n/2]
        ang = pos[:, axis].astype(np.float64)[:, None] * w   # [tokens, n/2]
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        a = x[:, :, off:off + n:2]       # first element of each pair
        b = x[:, :, off + 1:off + n:2]   # second element of each pair
        out[:, :, off:off + n:2] = a * c - b * s
        out[:, :, off + 1:off + n:2] = a * s + b * c
        off += n
    return out


def video_positions(frame0, n_frames, lat_h, lat_w):
    """(t, h, w) of every video token of frames [frame0, frame0+n_frames), raster order.

    Token index within a frame is h * lat_w + w.
    """
    f = np.arange(frame0, frame0 + n_frames, dtype=np.int64)
    hh, ww = np.meshgrid(np.arange(lat_h), np.arange(lat_w), indexing="ij")
    P = lat_h * lat_w
    t = np.repeat(f, P)
    h = np.tile(hh.reshape(-1), n_frames)
    w = np.tile(ww.reshape(-1), n_frames)
    return np.stack([t, h, w], axis=1)


def frame_positions(frames, lat_h, lat_w):
    """Positions of every token of an arbitrary list of absolute frames, in list order."""
    parts = [video_positions(int(f), 1, lat_h, lat_w) for f in frames]
    if not parts:
        return np.zeros((0, 3), dtype=np.int64)
    return np.concatenate(parts, axis=0)


def text_positions(n_text):
    """Text tokens sit at (0, 0, 0): no rotation."""
    return np.zeros((n_text, 3), dtype=np.int64)
