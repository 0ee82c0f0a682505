"""Dense softmax attention over a segment's key set, in fp64 (oracle, test-only).

Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
(ai.thesatyajit.com), sections "How one segment is made" (the current
segment's text and video tokens meet in joint attention; attention is
segment-wise causal, reading earlier segments from the KV cache; 16 heads of
128) and "What 'world memory' stores" (the cache holds, per layer, the keys and
values of earlier segments' tokens).

At inference only the newest segment has queries, so the segment-wise causal
mask reduces to: every query of the current segment sees every cached key and
every key of its own segment, with no mask inside the segment.

Readings where the pages are silent: softmax scale 1/sqrt(head_dim), no
query/key normalisation; query rows are the video tokens in (t, h, w) raster
order followed by the text tokens; keys are the kept history frames in list
order, then the current segment's frames, then its text tokens (the order of
keys does not change the result).
"""

import numpy as np

from .rope import rope3d


def attention(q, k, v, scale, visible=None):
    """Plain softmax attention for one head: softmax(scale * q k^T) v.

    q [M, D], k [N, D], v [N, D], all float64. Returns (out [M, D], lse [M]),
    lse = natural log of sum_j exp(scale * q.k_j). Exact row max first, then
    the sums (two passes). N == 0 is rejected: softmax over nothing is
    undefined. `visible` [M, N] (bool, optional) drops the keys a row may not
    see: their logits become -inf; a row that sees no key is rejected.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        raise ValueError("attention over an empty key set is undefined")
    s = (q @ k.T) * scale
    if visible is not None:
        visible = np.asarray(visible, dtype=bool)
        if not np.all(visible.any(axis=1)):
            raise ValueError("a query row sees no key")
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    lsum = p.sum(axis=1, keepdims=True)
    out = (p @ v) / lsum
    lse = (m + np.log(lsum))[:, 0]
    return out, lse


def timed_text_visibility(q_frame, key_text, window):
    """Which keys each query row may see under timed text windows.

    The pages (same article, "How one segment is made") give a second mask
    beside the segment-wise causal one: the text of an action that carries a
    time window is hidden from the video frames outside it, so the action is
    not acted out early. Reading (the window encoding is not on the
    pages): text token j carries an inclusive latent-frame range
    window[j] = (first, last); a video query in frame t sees it iff
    first <= t <= last; text queries and every non-text key are unaffected.

    q_frame  [M] latent frame of each query row, negative for text rows
    key_text [N] text-token index of each key, negative for video keys
    window   [n_text, 2] int
    Returns bool [M, N].
    """
    q_frame = np.asarray(q_frame, dtype=np.int64)
    key_text = np.asarray(key_text, dtype=np.int64)
    window = np.asarray(window, dtype=np.int64).reshape(-1, 2)
    is_text = key_text >= 0
    lo = np.where(is_text, window[np.maximum(key_text, 0), 0], 0)
    hi = np.where(is_text, window[np.maximum(key_text, 0), 1], 0)
    video_row = q_frame[:, None] >= 0
    inside = (lo[None, :] <= q_frame[:, None]) & (q_frame[:, None] <= hi[None, :])
    return ~is_text[None, :] | ~video_row | inside


def segment_attention(q, q_pos, k, k_pos, v, split=(16, 56, 56), theta=10000.0,
                      scale=None, rows=None, chunk=1024, q_frame=None, key_text=None,
                      text_window=None, block_lists=None, n_hist_frames=0, P=None):
    """Joint attention of one session over its key set, every head.

    q     [Lq, H, D]  raw (unrotated) queries, float64 (exact bf16 values)
    q_pos [Lq, 3]     (t, h, w) of each query row (text rows at 0, 0, 0)
    k, v  [Lk, H, D]  raw keys / values of the whole key set (kept history
                      frames, the own segment, the own text), float64
    k_pos [Lk, 3]     positions of the keys
    rows  optional index array of query rows to evaluate (sampling)
    q_frame, key_text, text_window: optional timed text windows
          (timed_text_visibility); all three or none
    block_lists, n_hist_frames, P: optional block-sparse history
          (sparse.sparse_visibility): block_lists [H, n_qblocks, keep] of kept
          candidate blocks over the first n_hist_frames frames (P tokens each)
          of the key set
    Returns (out [len(rows), H, D], lse [len(rows), H]).
    """
    from .sparse import sparse_visibility
    q = np.asarray(q, dtype=np.float64)
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        rows = np.arange(q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    qr = rope3d(q[rows], np.asarray(q_pos)[rows], split, theta)
    kr = rope3d(k, k_pos, split, theta)
    v = np.asarray(v, dtype=np.float64)
    H = q.shape[1]
    out = np.zeros((len(rows), H, D))
    lse = np.zeros((len(rows), H))
    for h in range(H):
        kh = np.ascontiguousarray(kr[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for c0 in range(0, len(rows), chunk):
            vis = None
            if text_window is not None:
                vis = timed_text_visibility(np.asarray(q_frame)[rows[c0:c0 + chunk]], key_text,
                                            text_window)
            if block_lists is not None:
                sv = sparse_visibility(rows[c0:c0 + chunk], block_lists[h], n_hist_frames, P,
                                       kh.shape[0])
                vis = sv if vis is None else (vis & sv)
            o, l = attention(qr[c0:c0 + chunk, h, :], kh, vh, scale, vis)
            out[c0:c0 + chunk, h, :] = o
            lse[c0:c0 + chunk, h] = l
    return out, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine attention over disjoint key sets A and B from their (out, lse).

    The identity the split/merge check relies on: with weights exp(lse_x - lse),
    lse = log(exp(lse_a) + exp(lse_b)), out = sum_x w_x * out_x.
    """
    m = np.maximum(lse_a, lse_b)
    wa = np.exp(lse_a - m)
    wb = np.exp(lse_b - m)
    lse = m + np.log(wa + wb)
    out = (o_a * wa[..., None] + o_b * wb[..., None]) / (wa + wb)[..., None]
    return out, lse
