"""Shared test helpers: build sessions through the HIP library and compute the
oracle's answer for the same seeded raw inputs.

The oracle only ever sees the raw bf16 inputs drawn by seeded_inputs (never a
value produced by the HIP library).
"""

import math

import numpy as np
import torch

import seeded_inputs as si
from oracle import attention as oatt
from oracle import numerics as onum
from oracle import rope as orope
from oracle import select as osel


def geom_for(wl, theta=None):
    import diffusion_transformer_attention_segment_amd as sa
    return sa.Geom(heads=wl.heads, lat_h=wl.lat_h, lat_w=wl.lat_w, rope_split=wl.split,
                   rope_theta=wl.theta if theta is None else theta)


def kept_frames(wl, session):
    """Kept history frames of a session (absolute indices), per the workload's policy."""
    T = wl.prior_segments[session] * wl.lat_t
    if wl.policy == "all":
        return osel.select_all(T).tolist()
    if wl.policy == "anchor_recent":
        return osel.select_anchor_recent(T, wl.lat_t, wl.recent_segments).tolist()
    raise ValueError(wl.policy)


def prob_rounding_bound(p, absv):
    """Per-element bound of the error that rounding the probabilities to e4m3
    adds to softmax(.) v: sum_j e_j |v_jd| / sum_j p_j, with p [M, N] the
    probabilities relative to each row's max (exp(s - max)) and absv [N, D].
    The e4m3 kernel weighs V by P' >= 2^5 p (its running max never passes the
    row's max by a whole unit), so a key with p >= 2^-11 has a normal P' and
    e = 2^-4 p (half a spacing at 3 mantissa bits); a smaller one may be
    subnormal, where half a spacing is 2^-10 in P' units, at most 2^-15 in p
    units, and rounding never moves a value by more than itself:
    e = max(2^-4 p, min(p, 2^-15)). Hidden keys have p = 0."""
    small = np.maximum(2.0 ** -4 * p, np.minimum(p, 2.0 ** -15))
    e = np.where(p >= 2.0 ** -11, 2.0 ** -4 * p, small)
    return (e @ absv) / p.sum(1)[:, None]


class Session:
    """One session of one layer: raw inputs on the device plus its cache layer."""

    def __init__(self, wl, seed, layer, session, device="cuda", theta=None, q_scale=1.0,
                 history=None):
        import diffusion_transformer_attention_segment_amd as sa
        self.wl, self.seed, self.layer_idx, self.session = wl, seed, layer, session
        self.geom = geom_for(wl, theta)
        S = wl.prior_segments[session]
        F = wl.lat_t
        self.S = S
        dtype = {"fp8": sa.KV_FP8, "int8": sa.KV_INT8}.get(wl.kv_dtype, sa.KV_BF16)
        text_cap = ((wl.n_text + 15) // 16) * 16
        self.kv = sa.KVLayer.allocate(self.geom, dtype, wl.frame_capacity(session), text_cap, device)
        self.raw_k, self.raw_v = [], []
        for seg in range(S + 1):
            k, v = si.segment_kv(wl, seed, layer, session, seg, device)
            self.raw_k.append(k)
            self.raw_v.append(v)
        self.text_k, self.text_v = si.text_kv(wl, seed, layer, session, device)
        q = si.queries(wl, seed, layer, session, device)
        if q_scale != 1.0:
            q = (q.float() * q_scale).to(torch.bfloat16)
        self.q = q
        for seg in range(S + 1):
            sa.kv_append(self.geom, self.kv, self.raw_k[seg], self.raw_v[seg], seg * F, F)
        sa.text_append(self.geom, self.kv, self.text_k, self.text_v, wl.n_text)
        hist = kept_frames(wl, session) if history is None else list(history)
        self.frames = hist + list(range(S * F, S * F + F))
        self.d_frames = torch.tensor(self.frames, dtype=torch.int32, device=device)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((wl.Lq, wl.heads), dtype=torch.float32, device=device)
        self.text_window = None      # timed text windows (set_windows)
        self.d_window = None
        self.block_lists = None      # block-sparse history (set_sparse)
        self.d_lists = None
        self.n_hist = 0

    def set_windows(self, win):
        """Timed text windows: int32 [n_text, 2] (first, last) absolute frames."""
        self.text_window = np.asarray(win, dtype=np.int64).reshape(-1, 2)
        self.d_window = torch.as_tensor(np.asarray(win, dtype=np.int32)).to(self.q.device).contiguous()

    def set_sparse(self, lists, n_hist):
        """Block-sparse history: int32 [H, n_qblocks, keep] kept candidate
        blocks over the first n_hist frames of the key set."""
        self.block_lists = np.asarray(lists, dtype=np.int32)
        self.d_lists = torch.as_tensor(self.block_lists).to(self.q.device).contiguous()
        self.n_hist = n_hist

    def clear_sparse(self):
        self.block_lists, self.d_lists, self.n_hist = None, None, 0

    def q_rotated(self):
        """Rotated queries (fp64) of every row: [Lq, H, D]."""
        wl = self.wl
        q = self.q.float().cpu().double().numpy()
        return orope.rope3d(q, self.q_positions(), wl.split, self.geom.rope_theta)

    def hist_stored_keys(self, n_hist):
        """Keys of the first n_hist frames of the key set as the cache stores
        them (the oracle's own append: rotated, bf16-rounded or e4m3 codes
        times the plane scale), fp64 [n_hist * P, H, D]."""
        from oracle import cache as ocache
        wl = self.wl
        F, P = wl.lat_t, wl.P
        out = []
        for f in self.frames[:n_hist]:
            seg, fo = divmod(f, F)
            raw = self.raw_k[seg][fo * P:(fo + 1) * P].float().cpu().double().numpy()
            if wl.kv_dtype == "fp8":
                kc, ksc, _, _ = ocache.append_fp8(raw, raw, f, wl.lat_h, wl.lat_w, wl.split,
                                                  self.geom.rope_theta)
                k = ocache.dequant(kc[0], ksc[0][:, None, None])
            elif wl.kv_dtype == "int8":
                kc, ksc, _, _ = ocache.append_int8(raw, raw, f, wl.lat_h, wl.lat_w, wl.split,
                                                   self.geom.rope_theta)
                k = ocache.dequant_int8(kc[0], ksc[0][..., None])
            else:
                k = ocache.append_bf16(raw, raw, f, wl.lat_h, wl.lat_w, wl.split,
                                       self.geom.rope_theta)[0][0]
            out.append(k.transpose(1, 0, 2))
        return np.concatenate(out)

    def oracle_select(self, n_hist, keep):
        """(lists [H, n_qblocks, keep], scores [H, n_qblocks, n_cand]) of the oracle."""
        from oracle import sparse as osp
        qr = self.q_rotated()
        kh = self.hist_stored_keys(n_hist)
        return (osp.select_blocks(qr, kh, n_hist, self.wl.P, keep),
                osp.block_scores(qr, kh, n_hist, self.wl.P))

    def q_frames(self):
        """Absolute latent frame of each query row, -1 for text rows."""
        wl = self.wl
        vid = self.S * wl.lat_t + np.arange(wl.lat_t * wl.P) // wl.P
        return np.concatenate([vid, -np.ones(wl.n_text, dtype=np.int64)])

    def key_text(self):
        """Text index of each key of the key set, -1 for video keys."""
        return np.concatenate([-np.ones(len(self.frames) * self.wl.P, dtype=np.int64),
                               np.arange(self.wl.n_text)])

    def visibility(self, rows, head=0):
        """bool [len(rows), Lk]: keys each row of `head` sees (None: all)."""
        from oracle import sparse as osp
        vis = None
        if self.text_window is not None:
            vis = oatt.timed_text_visibility(self.q_frames()[rows], self.key_text(), self.text_window)
        if self.block_lists is not None:
            sv = osp.sparse_visibility(rows, self.block_lists[head], self.n_hist, self.wl.P, self.Lk)
            vis = sv if vis is None else (vis & sv)
        return vis

    def item(self, with_lse=True):
        import diffusion_transformer_attention_segment_amd as sa
        wl = self.wl
        return sa.AttnItem(self.q, self.kv, self.d_frames, len(self.frames), wl.n_text, self.out,
                           frame0_q=self.S * wl.lat_t, n_frames_q=wl.lat_t, n_text_q=wl.n_text,
                           lse=self.lse if with_lse else None, text_window=self.d_window,
                           block_list=self.d_lists, n_hist_frames=self.n_hist,
                           keep_blocks=0 if self.block_lists is None else self.block_lists.shape[2])

    @property
    def Lk(self):
        return len(self.frames) * self.wl.P + self.wl.n_text

    # ---------------------------------------------------------------- oracle
    def raw_keys(self, heads=None):
        """Raw K, V (float64) of the whole key set and their positions, host side."""
        wl = self.wl
        F, P = wl.lat_t, wl.P
        hs = slice(None) if heads is None else list(heads)
        ks, vs = [], []
        for f in self.frames:
            seg, fo = divmod(f, F)
            ks.append(self.raw_k[seg][fo * P:(fo + 1) * P][:, hs])
            vs.append(self.raw_v[seg][fo * P:(fo + 1) * P][:, hs])
        ks.append(self.text_k[:, hs])
        vs.append(self.text_v[:, hs])
        k = torch.cat(ks).float().cpu().double().numpy()
        v = torch.cat(vs).float().cpu().double().numpy()
        pos = np.concatenate([orope.frame_positions(self.frames, wl.lat_h, wl.lat_w),
                              orope.text_positions(wl.n_text)])
        return k, v, pos

    def q_positions(self):
        wl = self.wl
        return np.concatenate([orope.video_positions(self.S * wl.lat_t, wl.lat_t, wl.lat_h, wl.lat_w),
                               orope.text_positions(wl.n_text)])

    def oracle(self, rows=None, heads=None, round_rotated=False):
        """Oracle (out, lse) for the given rows and heads.

        round_rotated=True is the diagnostic variant: it models the bf16
        operands of the kernel -- rotated keys rounded to bf16 (the cache) and
        rotated queries times scale * log2(e) rounded to bf16 (the query
        operand carries the softmax scale in log2 units) -- before the fp64
        attention, so what remains is the kernel's own arithmetic error.
        """
        wl = self.wl
        k, v, kpos = self.raw_keys(heads)
        hs = slice(None) if heads is None else list(heads)
        q = self.q[:, hs].float().cpu().double().numpy()
        scale = 1.0 / math.sqrt(wl.head_dim)
        win = {}
        if self.text_window is not None:
            win = dict(q_frame=self.q_frames(), key_text=self.key_text(),
                       text_window=self.text_window)
        if self.block_lists is not None:
            hl = self.block_lists if heads is None else self.block_lists[list(heads)]
            win.update(block_lists=hl, n_hist_frames=self.n_hist, P=wl.P)
        if not round_rotated:
            return oatt.segment_attention(q, self.q_positions(), k, kpos, v, wl.split,
                                          self.geom.rope_theta, scale, rows=rows, **win)
        if rows is None:
            rows = np.arange(q.shape[0])
        hsel = list(range(wl.heads)) if heads is None else list(heads)
        c2 = float(np.float32(scale * math.log2(math.e)))
        qr = onum.bf16_round(orope.rope3d(q[rows], self.q_positions()[rows], wl.split,
                                          self.geom.rope_theta) * c2) / c2
        kr = onum.bf16_round(orope.rope3d(k, kpos, wl.split, self.geom.rope_theta))
        out = np.zeros(qr.shape)
        lse = np.zeros(qr.shape[:2])
        for h in range(qr.shape[1]):
            out[:, h], lse[:, h] = oatt.attention(qr[:, h], kr[:, h], v[:, h], scale,
                                                  self.visibility(rows, hsel[h]))
        return out, lse

    def fp8_stored_kv(self, hs):
        """The key set of heads hs as an e4m3 cache stores it, from the
        oracle's own append (quantise, then decode times the plane scale):
        rotated K [Lk, len(hs), D] and V [Lk, len(hs), D], float64."""
        from oracle import cache as ocache
        wl = self.wl
        F, P = wl.lat_t, wl.P
        raw = [(f, self.raw_k[f // F][(f % F) * P:(f % F + 1) * P].float().cpu().double().numpy(),
                self.raw_v[f // F][(f % F) * P:(f % F + 1) * P].float().cpu().double().numpy())
               for f in self.frames]

        def one_frame(args):     # the oracle's own append and decode of one frame
            f, kin, vin = args
            kc, ksc, vc, vsc = ocache.append_fp8(kin, vin, f, wl.lat_h, wl.lat_w, wl.split,
                                                 self.geom.rope_theta)
            return (ocache.dequant(kc[0], ksc[0][:, None, None]).transpose(1, 0, 2)[:, hs],
                    ocache.dequant(vc[0], vsc[0][:, None, None]).transpose(2, 0, 1)[:, hs])

        import concurrent.futures   # frames are independent: one per worker thread
        with concurrent.futures.ThreadPoolExecutor(max_workers=16) as ex:
            per_frame = list(ex.map(one_frame, raw))
        del raw
        ks = [x[0] for x in per_frame]
        vs = [x[1] for x in per_frame]
        del per_frame
        tk = self.text_k.float().cpu().double().numpy()
        tv = self.text_v.float().cpu().double().numpy()
        kc, ksc, vc, vsc = ocache.append_text_fp8(tk, tv)
        ks.append(ocache.dequant(kc, ksc[:, None, None]).transpose(1, 0, 2)[:, hs])
        vs.append(ocache.dequant(vc, vsc[:, None, None]).transpose(2, 0, 1)[:, hs])
        k = np.concatenate(ks)          # already rotated
        v = np.concatenate(vs)
        return k, v

    def oracle_fp8_cache(self, rows=None, heads=None, split_q=False):
        """Oracle for an e4m3 cache: fp64 attention over the values the cache
        stores -- the oracle's own quantised-then-dequantised K and V (per
        (frame, head) planes, per head for text) -- and the fp64 rotated Q.
        split_q=True is the diagnostic variant that also models the kernel's
        query precision (split_query_fp8).

        Returns (out, lse, bound): `bound` is the per-element error that rounding
        the probabilities to e4m3 can add (prob_rounding_bound: the kernel
        multiplies V by e4m3 probabilities P' = 2^(x - m + 6) against its
        running max m)."""
        wl = self.wl
        hs = list(range(wl.heads)) if heads is None else list(heads)
        k, v = self.fp8_stored_kv(hs)
        q = self.q[:, hs].float().cpu().double().numpy()
        if rows is None:
            rows = np.arange(q.shape[0])
        qr = orope.rope3d(q[rows], self.q_positions()[rows], wl.split, self.geom.rope_theta)
        qq = qr.copy()
        scale = 1.0 / math.sqrt(wl.head_dim)
        if split_q:
            for i in range(qr.shape[0]):
                for j in range(qr.shape[1]):
                    qq[i, j] = split_query_fp8(qr[i, j], np.float32(scale * math.log2(math.e)))
        out = np.zeros(qq.shape)
        lse = np.zeros(qq.shape[:2])
        bound = np.zeros(qq.shape)
        for j in range(qq.shape[1]):
            vis = self.visibility(rows, hs[j])
            out[:, j], lse[:, j] = oatt.attention(qq[:, j], k[:, j], v[:, j], scale, vis)
            s_ = (qq[:, j] @ k[:, j].T) * scale
            if vis is not None:
                s_ = np.where(vis, s_, -np.inf)
            p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
            bound[:, j] = prob_rounding_bound(p_, np.abs(v[:, j]))
        return out, lse, bound

    def oracle_int8_cache(self, rows=None, heads=None):
        """Oracle for an int8 cache: fp64 attention over the values the cache
        stores (the oracle's own per-token int8 quantisation of rotated K and
        of V, times the scales) and the fp64 rotated Q. Returns (out, lse)."""
        from oracle import cache as ocache
        wl = self.wl
        hs = list(range(wl.heads)) if heads is None else list(heads)
        F, P = wl.lat_t, wl.P
        ks, vs = [], []
        for f in self.frames:
            seg, fo = divmod(f, F)
            kin = self.raw_k[seg][fo * P:(fo + 1) * P][:, hs].float().cpu().double().numpy()
            vin = self.raw_v[seg][fo * P:(fo + 1) * P][:, hs].float().cpu().double().numpy()
            kc, ksc, vc, vsc = ocache.append_int8(kin, vin, f, wl.lat_h, wl.lat_w, wl.split,
                                                  self.geom.rope_theta)
            ks.append(ocache.dequant_int8(kc[0], ksc[0][..., None]).transpose(1, 0, 2))
            vs.append(ocache.dequant_int8(vc[0], vsc[0][:, None, :]).transpose(2, 0, 1))
        tk = self.text_k[:, hs].float().cpu().double().numpy()
        tv = self.text_v[:, hs].float().cpu().double().numpy()
        kc, ksc, vc, vsc = ocache.append_text_int8(tk, tv)
        ks.append(ocache.dequant_int8(kc, ksc[..., None]).transpose(1, 0, 2))
        vs.append(ocache.dequant_int8(vc, vsc[:, None, :]).transpose(2, 0, 1))
        k = np.concatenate(ks)          # already rotated
        v = np.concatenate(vs)
        q = self.q[:, hs].float().cpu().double().numpy()
        if rows is None:
            rows = np.arange(q.shape[0])
        qr = orope.rope3d(q[rows], self.q_positions()[rows], wl.split, self.geom.rope_theta)
        scale = 1.0 / math.sqrt(wl.head_dim)
        out = np.zeros(qr.shape)
        lse = np.zeros(qr.shape[:2])
        for j in range(qr.shape[1]):
            out[:, j], lse[:, j] = oatt.attention(qr[:, j], k[:, j], v[:, j], scale,
                                                  self.visibility(rows, hs[j]))
        return out, lse

    def gpu_out(self, rows=None, heads=None):
        o = self.out.float().cpu().double().numpy()
        l = self.lse.cpu().double().numpy()
        if rows is not None:
            o, l = o[rows], l[rows]
        if heads is not None:
            o, l = o[:, list(heads)], l[:, list(heads)]
        return o, l


def oracle_all_heads(s, rows=None, workers=16):
    """Session.oracle over every head, one head per worker thread (the
    oracle's numpy calls release the interpreter lock; BLAS is held to one
    thread per worker). Same arithmetic as s.oracle(rows): the heads are
    independent. Prints a line per finished head."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    wl = s.wl
    k, v, kpos = s.raw_keys()
    q = s.q.float().cpu().double().numpy()
    qpos = s.q_positions()
    scale = 1.0 / math.sqrt(wl.head_dim)
    n = q.shape[0] if rows is None else len(rows)
    out = np.zeros((n, wl.heads, wl.head_dim))
    lse = np.zeros((n, wl.heads))

    def one(h):
        o, l = oatt.segment_attention(q[:, h:h + 1], qpos, k[:, h:h + 1], kpos, v[:, h:h + 1],
                                      wl.split, s.geom.rope_theta, scale, rows=rows)
        out[:, h] = o[:, 0]
        lse[:, h] = l[:, 0]
        print(f"  oracle head {h} done", flush=True)

    with threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(wl.heads)))
    return out, lse


def oracle_fp8_cache_all_heads(s, rows=None, workers=16, chunk=256, with_bound=False):
    """Session.oracle_fp8_cache's (out, lse) for every head: the oracle over
    the values an e4m3 cache stores, one head per worker thread, query rows in
    chunks of `chunk` so that a full-size output fits in memory. With
    with_bound, also the e4m3 probability-rounding bound of
    Session.oracle_fp8_cache and each row's largest probability (out, lse,
    bound, pmax). Prints a line per finished head."""
    import concurrent.futures
    from threadpoolctl import threadpool_limits
    wl = s.wl
    k, v = s.fp8_stored_kv(list(range(wl.heads)))
    q = s.q.float().cpu().double().numpy()
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    qr = orope.rope3d(q[rows], s.q_positions()[rows], wl.split, s.geom.rope_theta)
    scale = 1.0 / math.sqrt(wl.head_dim)
    out = np.zeros(qr.shape)
    lse = np.zeros(qr.shape[:2])
    bound = np.zeros(qr.shape) if with_bound else None
    pmax = np.zeros(qr.shape[:2]) if with_bound else None

    def one(h):
        kh = np.ascontiguousarray(k[:, h])
        vh = np.ascontiguousarray(v[:, h])
        for c0 in range(0, len(rows), chunk):
            vis = s.visibility(rows[c0:c0 + chunk], h)
            o, l = oatt.attention(qr[c0:c0 + chunk, h], kh, vh, scale, vis)
            out[c0:c0 + chunk, h] = o
            lse[c0:c0 + chunk, h] = l
            if with_bound:   # as Session.oracle_fp8_cache's bound
                s_ = (qr[c0:c0 + chunk, h] @ kh.T) * scale
                if vis is not None:
                    s_ = np.where(vis, s_, -np.inf)
                p_ = np.exp(s_ - s_.max(axis=1, keepdims=True))
                bound[c0:c0 + chunk, h] = prob_rounding_bound(p_, np.abs(vh))
                pmax[c0:c0 + chunk, h] = 1.0 / p_.sum(1)
        print(f"  oracle head {h} done", flush=True)

    with threadpool_limits(1):
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, range(wl.heads)))
    if with_bound:
        return out, lse, bound, pmax
    return out, lse


def split_query_fp8(q, scale_log2):
    """Real value of a rotated query row as the e4m3 kernel takes it: in fp32,
    x = q * scale_log2 (softmax scale times log2(e)), amax = max |x|, the
    power of two 2^qe with amax <= 448 * 2^qe (at least 2^-122), y = x * 2^-qe,
    hi = e4m3(y), lo = e4m3(16 (y - hi)); value (hi + lo / 16) 2^qe / scale_log2."""
    x = (np.asarray(q, dtype=np.float64).astype(np.float32) * np.float32(scale_log2)).astype(np.float64)
    amax = float(np.max(np.abs(x)))
    if amax == 0:
        return np.zeros(x.shape)
    qe = -122
    while amax > 448.0 * 2.0 ** qe:
        qe += 1
    y = x * 2.0 ** -qe
    hi = onum.e4m3_decode(onum.e4m3_encode(y))
    lo = onum.e4m3_decode(onum.e4m3_encode(16.0 * (y - hi)))
    return (hi + lo / 16.0) * 2.0 ** qe / float(np.float32(scale_log2))


def compare(got, want, max_abs, mean_abs, label=""):
    err = np.abs(got - want)
    mx, mn = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    msg = f"{label}: max_abs={mx:.3e} mean_abs={mn:.3e} rel_l2={rel:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), msg
    assert mx <= max_abs and mn <= mean_abs, msg
    return mx, mn, rel


def check_block_lists(got, want, scores, rel_tol):
    """GPU lists vs oracle lists: equal up to near-ties at the threshold."""
    H, nq, keep = want.shape
    assert got.shape == want.shape
    n_cand = scores.shape[2]
    swaps = 0
    for h in range(H):
        for i in range(nq):
            g = got[h, i]
            assert np.all(np.diff(g) > 0) and g[0] >= 0 and g[-1] < n_cand, (h, i, g)
            diff = set(g.tolist()) ^ set(want[h, i].tolist())
            if not diff:
                continue
            sc = scores[h, i]
            thr = np.sort(sc)[::-1][keep - 1]
            tol = rel_tol * np.abs(sc).max()
            for b in diff:
                assert abs(sc[b] - thr) <= tol, (h, i, b, sc[b], thr)
            swaps += len(diff) // 2
    return swaps
