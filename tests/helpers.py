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
        dtype = sa.KV_FP8 if wl.kv_dtype == "fp8" else sa.KV_BF16
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

    def item(self, with_lse=True):
        import diffusion_transformer_attention_segment_amd as sa
        wl = self.wl
        return sa.AttnItem(self.q, self.kv, self.d_frames, len(self.frames), wl.n_text, self.out,
                           frame0_q=self.S * wl.lat_t, n_frames_q=wl.lat_t, n_text_q=wl.n_text,
                           lse=self.lse if with_lse else None)

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

        round_rotated=True is the diagnostic variant: rotated queries and keys
        are rounded to bf16 before the fp64 attention, modelling the documented
        storage of rotated keys in a bf16 cache and the bf16 MFMA operands, so
        what remains is the kernel's own arithmetic error.
        """
        wl = self.wl
        k, v, kpos = self.raw_keys(heads)
        hs = slice(None) if heads is None else list(heads)
        q = self.q[:, hs].float().cpu().double().numpy()
        scale = 1.0 / math.sqrt(wl.head_dim)
        if not round_rotated:
            return oatt.segment_attention(q, self.q_positions(), k, kpos, v, wl.split,
                                          self.geom.rope_theta, scale, rows=rows)
        if rows is None:
            rows = np.arange(q.shape[0])
        qr = onum.bf16_round(orope.rope3d(q[rows], self.q_positions()[rows], wl.split,
                                          self.geom.rope_theta))
        kr = onum.bf16_round(orope.rope3d(k, kpos, wl.split, self.geom.rope_theta))
        out = np.zeros(qr.shape)
        lse = np.zeros(qr.shape[:2])
        for h in range(qr.shape[1]):
            out[:, h], lse[:, h] = oatt.attention(qr[:, h], kr[:, h], v[:, h], scale)
        return out, lse

    def gpu_out(self, rows=None, heads=None):
        o = self.out.float().cpu().double().numpy()
        l = self.lse.cpu().double().numpy()
        if rows is not None:
            o, l = o[rows], l[rows]
        if heads is not None:
            o, l = o[:, list(heads)], l[:, list(heads)]
        return o, l


def compare(got, want, max_abs, mean_abs, label=""):
    err = np.abs(got - want)
    mx, mn = float(err.max()), float(err.mean())
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    msg = f"{label}: max_abs={mx:.3e} mean_abs={mn:.3e} rel_l2={rel:.3e}"
    print(msg, flush=True)
    assert np.all(np.isfinite(got)), msg
    assert mx <= max_abs and mn <= mean_abs, msg
    return mx, mn, rel
