"""Block-sparse history attention: block selection and visibility (oracle, test-only).

Source: "Hy-Nomas en una RTX 4090" (inferencekey.com), section "El preset de
una GPU": citing the technical report (its section 6.2), the single-GPU preset
adds sparse attention that is dense in the first two denoising steps and then
keeps 25 % of the candidate video blocks. The pages give neither the block
size nor the selection rule. Readings taken here (plainest ones):

- candidates: the keys of the kept history frames (the frames cached before
  the current segment), cut per frame into blocks of 64 consecutive tokens
  (the last block of a frame is shorter when 64 does not divide the frame);
  block b of frame-list position f and in-frame index j is b = f * ceil(P / 64)
  + j. The current segment's frames and the text keys are always attended;
- query blocks: 256 consecutive query rows in token order (video raster
  order, then text), the last one shorter;
- score of (query block, candidate block), per head: the mean of the block's
  rotated queries dotted with the mean of the block's stored (rotated) keys;
- keep = ceil(n_candidates * percent / 100) candidates with the highest
  scores, ties to the lower block index, per (head, query block); the list is
  stored in ascending block order;
- whether a pass is dense or sparse (the first two steps dense) is the
  caller's choice.

Everything here is plain numpy in fp64.
"""

import math

import numpy as np

KEY_BLOCK = 64
QUERY_BLOCK = 256


def keep_count(n_candidates, percent):
    """Blocks kept out of n_candidates at `percent` (ceil, at most all)."""
    if n_candidates <= 0:
        return 0
    return min(n_candidates, max(1, math.ceil(n_candidates * percent / 100.0)))


def candidate_blocks(n_hist_frames, P, block=KEY_BLOCK):
    """(frame position, first token in frame, length) of every candidate, in block order."""
    per = -(-P // block)
    out = []
    for f in range(n_hist_frames):
        for j in range(per):
            s = j * block
            out.append((f, s, min(block, P - s)))
    return out


def pooled_keys(k_hist, n_hist_frames, P, block=KEY_BLOCK):
    """Mean key of each candidate block. k_hist [n_hist_frames * P, H, D]
    (stored rotated keys, frame-list order) -> [H, n_candidates, D]."""
    k_hist = np.asarray(k_hist, dtype=np.float64)
    blocks = candidate_blocks(n_hist_frames, P, block)
    H, D = k_hist.shape[1], k_hist.shape[2]
    out = np.zeros((H, len(blocks), D))
    for b, (f, s, n) in enumerate(blocks):
        out[:, b, :] = k_hist[f * P + s:f * P + s + n].mean(axis=0)
    return out


def pooled_queries(q_rot, block_q=QUERY_BLOCK):
    """Mean rotated query of each query block. q_rot [Lq, H, D] -> [H, n_qblocks, D]."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    Lq, H, D = q_rot.shape
    nb = -(-Lq // block_q)
    out = np.zeros((H, nb, D))
    for i in range(nb):
        out[:, i, :] = q_rot[i * block_q:min(Lq, (i + 1) * block_q)].mean(axis=0)
    return out


def block_scores(q_rot, k_hist, n_hist_frames, P, block=KEY_BLOCK, block_q=QUERY_BLOCK):
    """Scores [H, n_qblocks, n_candidates]: pooled query . pooled key."""
    pq = pooled_queries(q_rot, block_q)
    pk = pooled_keys(k_hist, n_hist_frames, P, block)
    return np.einsum("hqd,hcd->hqc", pq, pk)


def select_blocks(q_rot, k_hist, n_hist_frames, P, keep, block=KEY_BLOCK, block_q=QUERY_BLOCK):
    """Kept candidate blocks: int32 [H, n_qblocks, keep], ascending per list.

    Highest score first, ties to the lower block index; the kept indices are
    then listed in ascending order."""
    sc = block_scores(q_rot, k_hist, n_hist_frames, P, block, block_q)
    H, nq, nc = sc.shape
    out = np.zeros((H, nq, keep), dtype=np.int32)
    idx = np.arange(nc)
    for h in range(H):
        for i in range(nq):
            order = np.lexsort((idx, -sc[h, i]))     # primary: score desc; then index asc
            out[h, i] = np.sort(order[:keep])
    return out


def sparse_visibility(rows, lists_h, n_hist_frames, P, n_keys, block=KEY_BLOCK,
                      block_q=QUERY_BLOCK):
    """bool [len(rows), n_keys] for one head: keys of unkept candidate blocks are
    hidden from the rows of that query block; every other key is visible.

    lists_h [n_qblocks, keep]: kept blocks per query block of this head. Keys
    are ordered history frames (candidates) first, then the rest."""
    rows = np.asarray(rows, dtype=np.int64)
    blocks = candidate_blocks(n_hist_frames, P, block)
    n_cand_keys = n_hist_frames * P
    block_of_key = np.zeros(n_cand_keys, dtype=np.int64)
    for b, (f, s, n) in enumerate(blocks):
        block_of_key[f * P + s:f * P + s + n] = b
    vis = np.ones((len(rows), n_keys), dtype=bool)
    for r_i, r in enumerate(rows):
        kept = np.zeros(len(blocks), dtype=bool)
        kept[np.asarray(lists_h[r // block_q], dtype=np.int64)] = True
        vis[r_i, :n_cand_keys] = kept[block_of_key]
    return vis
