"""History frame selection policies (oracle, test-only).

Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
(ai.thesatyajit.com), section "The 4090 preset". The single-GPU preset keeps a
budget of past latent frames on the GPU, picked power-spaced back from the
newest frame:

    d_i = i + rint((T - N) * u_i ** gamma),  u_i = i / (N - 1),
    N = min(budget, T),  gamma = 2,

with T past latent frames; the kept frames are T - 1 - d_i. The page prints the
result for T = 360, budget 18.

Readings where the page is silent:

* T <= budget keeps every frame; N == 1 keeps the newest frame; T == 0 keeps
  nothing (the segment then attends to itself only);
* rint is round-half-to-even in float64, evaluated in the order written;
* the output is sorted ascending (oldest first).

Two further policies that the workloads use:

* RECENT(budget): the newest min(budget, T) frames (a true sliding window,
  which the page contrasts with the preset's pick);
* ANCHOR_RECENT(F, R): the first frame of every past segment of F frames plus
  every frame of the newest R segments.
"""

import numpy as np


def select_all(T):
    return np.arange(T, dtype=np.int64)


def select_recent(T, budget):
    n = min(budget, T)
    return np.arange(T - n, T, dtype=np.int64)


def select_power(T, budget, gamma=2.0):
    if T <= 0:
        return np.zeros(0, dtype=np.int64)
    N = min(budget, T)
    if N == T:
        return np.arange(T, dtype=np.int64)
    if N == 1:
        return np.array([T - 1], dtype=np.int64)
    picks = []
    for i in range(N):
        u = i / (N - 1)
        d = i + int(np.rint((T - N) * u ** gamma))
        picks.append(T - 1 - d)
    return np.array(sorted(picks), dtype=np.int64)


def select_anchor_recent(T, frames_per_segment, recent_segments):
    """First frame of each F-frame segment, plus all frames of the newest R segments."""
    F = frames_per_segment
    anchors = set(range(0, T, F))
    n_seg = -(-T // F)                      # segments touched by T frames
    first_recent_seg = max(0, n_seg - recent_segments)
    recent = set(range(first_recent_seg * F, T))
    return np.array(sorted(anchors | recent), dtype=np.int64)
