"""Seeded synthetic inputs for segment attention (shared by tests, smoke and bench).

This module only draws random numbers and describes workload shapes; it holds
none of the method's arithmetic (no rotation, no attention, no quantisation),
so both the HIP path and the CPU oracle may consume what it produces.

Workload shapes stand in for the pages' 5-second 720p segment
("Hy-Nomas: an 8.6B world model whose memory is a KV cache", section "How one
segment is made": 22 x 40 tokens per latent frame, 30 latent frames per
segment, 16 heads of 128). Values: raw Q, K, V ~ N(0, 1) in float32, rounded
to bf16 (round-nearest-even, by torch). The fp8 workload multiplies raw K and V
by independent factors U[0.5, 2] per (latent frame, head) before that rounding.
"""

from dataclasses import dataclass, field
import zlib

import torch

SPLIT = (16, 56, 56)


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    lat_t: int            # latent frames per segment (F)
    lat_h: int
    lat_w: int
    n_text: int
    prior_segments: tuple  # prior segments per session
    kv_dtype: str = "bf16"  # "bf16", "fp8" or "int8"
    layers: int = 1
    policy: str = "all"     # history policy: "all" or "anchor_recent"
    recent_segments: int = 3
    capacity_segments: int = 0   # 0: exactly prior + current
    theta: float = 10000.0
    head_dim: int = 128
    scale_factors: bool = False  # U[0.5, 2] per (frame, head) on K and V
    split: tuple = field(default=SPLIT)

    @property
    def P(self):
        return self.lat_h * self.lat_w

    @property
    def sessions(self):
        return len(self.prior_segments)

    def frame_capacity(self, session):
        segs = self.capacity_segments or (self.prior_segments[session] + 1)
        return segs * self.lat_t

    @property
    def Lq(self):
        return self.lat_t * self.P + self.n_text


def _config4_second_session(seed=0):
    g = torch.Generator().manual_seed(derive_seed(seed, "config4", "session1_len"))
    return int(torch.randint(4, 12, (1,), generator=g).item())   # 4..11 segments


def workloads(seed=0):
    """The workloads, in order: tiny, one prior segment, long history,
    active-history selection (2 sessions), fp8 cache, int8 cache (the pages'
    per-token format) over the same eight prior segments."""
    return [
        Workload("tiny", heads=2, lat_t=2, lat_h=4, lat_w=6, n_text=16,
                 prior_segments=(2,)),
        Workload("seg1", heads=16, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                 prior_segments=(1,)),
        Workload("seg4x54", heads=16, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                 prior_segments=(4,), layers=54),
        Workload("select2", heads=16, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                 prior_segments=(12, _config4_second_session(seed)),
                 policy="anchor_recent", capacity_segments=13),
        Workload("fp8seg8", heads=16, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                 prior_segments=(8,), kv_dtype="fp8", scale_factors=True),
        Workload("int8seg8", heads=16, lat_t=30, lat_h=22, lat_w=40, n_text=256,
                 prior_segments=(8,), kv_dtype="int8"),
    ]


def derive_seed(base, *parts):
    """Stable 63-bit seed from a base seed and a tuple of labels."""
    h = zlib.crc32(repr((int(base),) + tuple(parts)).encode())
    h2 = zlib.crc32(repr(tuple(parts) + (int(base), "x")).encode())
    return ((h << 31) ^ h2) & ((1 << 63) - 1)


def normal_bf16(shape, seed, device="cpu"):
    """N(0, 1) float32 draws rounded to bf16, from a torch generator seeded with ``seed``."""
    g = torch.Generator(device=device).manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def uniform_factors(shape, seed, lo=0.5, hi=2.0):
    """U[lo, hi] float32 factors on the CPU (small tensors)."""
    g = torch.Generator().manual_seed(int(seed))
    return lo + (hi - lo) * torch.rand(shape, generator=g, dtype=torch.float32)


def segment_kv(wl, seed, layer, session, segment, device="cpu"):
    """Raw K and V of one segment's video tokens: bf16 [F*P, H, D] each."""
    shape = (wl.lat_t * wl.P, wl.heads, wl.head_dim)
    out = []
    for kind in ("k", "v"):
        s = derive_seed(seed, wl.name, layer, session, segment, kind)
        if not wl.scale_factors:
            out.append(normal_bf16(shape, s, device))
            continue
        g = torch.Generator(device=device).manual_seed(int(s))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        fac = uniform_factors((wl.lat_t, wl.heads),
                              derive_seed(seed, wl.name, layer, session, segment,
                                          kind, "factor"))
        fac = fac.to(device).repeat_interleave(wl.P, dim=0)[:, :, None]
        out.append((x * fac).to(torch.bfloat16))
    return out[0], out[1]


def text_kv(wl, seed, layer, session, device="cpu"):
    """Raw K and V of the current segment's text tokens: bf16 [n_text, H, D]."""
    shape = (wl.n_text, wl.heads, wl.head_dim)
    out = []
    for kind in ("k", "v"):
        s = derive_seed(seed, wl.name, layer, session, "text", kind)
        if not wl.scale_factors:
            out.append(normal_bf16(shape, s, device))
            continue
        g = torch.Generator(device=device).manual_seed(int(s))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        fac = uniform_factors((wl.heads,), derive_seed(seed, wl.name, layer, session,
                                                       "text", kind, "factor"))
        out.append((x * fac.to(device)[None, :, None]).to(torch.bfloat16))
    return out[0], out[1]


def queries(wl, seed, layer, session, device="cpu"):
    """Raw queries of the current segment: bf16 [F*P + n_text, H, D] (video rows, then text)."""
    return normal_bf16((wl.Lq, wl.heads, wl.head_dim),
                       derive_seed(seed, wl.name, layer, session, "q"), device)


def sample_rows(n_rows, n_sample, seed, boundaries=()):
    """A seeded sample of row indices that always includes the first, last and
    the given boundary rows (clipped to range), sorted and unique."""
    g = torch.Generator().manual_seed(int(derive_seed(seed, "rows", n_rows, n_sample)))
    base = torch.randint(0, n_rows, (n_sample,), generator=g).tolist()
    extra = [0, n_rows - 1] + [b for b in boundaries if 0 <= b < n_rows]
    return sorted(set(base) | set(extra))


def text_windows(wl, seed, frame0, n_actions=4):
    """Timed text windows for the current segment's text tokens: int32
    [n_text, 2] of inclusive absolute latent frames (first, last).

    Recipe: the text tokens are cut at seeded points into n_actions contiguous
    spans (one prompt each). Span 0 is always on (frames 0 .. frame0 + F + 8);
    span 1 is off for the whole segment (a window entirely before frame0); the
    others get seeded windows [a, b] with frame0 - 2 <= a <= b <= frame0 + F + 1,
    so that most frames see some actions and not others."""
    n = wl.n_text
    F = wl.lat_t
    g = torch.Generator().manual_seed(int(derive_seed(seed, wl.name, "windows", frame0)))
    k = max(1, min(n_actions, n))
    cuts = sorted(torch.randperm(max(n - 1, 1), generator=g)[:k - 1].add(1).tolist()) if n > 1 else []
    bounds = [0] + cuts + [n]
    win = torch.zeros((n, 2), dtype=torch.int32)
    for i in range(len(bounds) - 1):
        if i == 0:
            lo, hi = 0, frame0 + F + 8
        elif i == 1:
            lo, hi = max(frame0 - 6, 0), max(frame0 - 3, 0) if frame0 >= 3 else -1
        else:
            a, b = torch.randint(frame0 - 2, frame0 + F + 2, (2,), generator=g).tolist()
            lo, hi = min(a, b), max(a, b)
        win[bounds[i]:bounds[i + 1], 0] = lo
        win[bounds[i]:bounds[i + 1], 1] = hi
    return win
