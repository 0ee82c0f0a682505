"""GPU parity on seeded random shapes, through the C ABI.

Each case draws its own geometry and key set from a seeded generator: 1-4
heads, latent grids from 2 x 4 to 9 x 16 (frames of 8 to 144 tokens, a
multiple of 8 as the library requires; padded planes for the one-byte
caches), 1-4 frames per segment, 0-257 text tokens,
0-3 prior segments whose kept frames are a random subset in random order (or
all of them, in order), timed text windows on half of the cases, split tiles
on half of the cases, and block-sparse history (1, 25, 50 or 100 % kept) on
some of the cases with a history: there the library's block lists are
checked against the oracle's selection, and the attention runs with the
oracle's lists. The cache type cycles through bf16, e4m3 (values
scaled per (frame, head)) and int8. Each output is checked against the
oracle for the same inputs with that cache type's bar: bf16 max-abs 2e-2,
mean-abs 2e-3, relative L2 1e-2; e4m3 per element within the e4m3
probability-rounding bound plus 5e-3 against the oracle over the stored
values, relative L2 0.05; int8 the bf16 bar against the oracle over the
stored values.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session, check_block_lists, compare

pytestmark = pytest.mark.gpu

KINDS = ("bf16", "fp8", "int8")
N_CASES = 48


def _draw(case):
    g = np.random.default_rng(si.derive_seed(0, "shape sweep", case))
    kv = KINDS[case % 3]
    H = int(g.integers(1, 5))
    while True:   # the library's limit: tokens per frame a multiple of 8
        lh, lw = int(g.integers(2, 10)), int(g.integers(2, 18))
        if lh * lw % 8 == 0:
            break
    F = int(g.integers(1, 5))
    n_text = int(g.choice([0, 1, 16, 37, 64, 100, 257]))
    prior = int(g.integers(0, 4))
    wl = si.Workload(f"sweep{case}", heads=H, lat_t=F, lat_h=lh, lat_w=lw, n_text=n_text,
                     prior_segments=(prior,), kv_dtype=kv, scale_factors=(kv == "fp8"))
    history = None
    if prior > 0 and g.random() < 0.7:
        n_keep = int(g.integers(1, prior * F + 1))
        history = [int(f) for f in g.choice(prior * F, size=n_keep, replace=False)]
    windows = n_text > 0 and g.random() < 0.5
    split = bool(g.random() < 0.5)
    # block-sparse history on some cases with a history: the kept percentage
    sparse = int(g.choice([1, 25, 50, 100])) if prior > 0 and g.random() < 0.4 else 0
    return wl, history, windows, split, sparse


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(case):
    wl, history, windows, split, sparse = _draw(case)
    label = (f"case {case}: {wl.kv_dtype} H={wl.heads} grid={wl.lat_h}x{wl.lat_w} F={wl.lat_t} "
             f"text={wl.n_text} prior={wl.prior_segments[0]} "
             f"history={'all' if history is None else len(history)} windows={windows} "
             f"split={split} sparse={sparse or 'no'}")
    print(label, flush=True)
    s = Session(wl, seed=case, layer=0, session=0, history=history)
    if windows:
        s.set_windows(si.text_windows(wl, case, wl.prior_segments[0] * wl.lat_t))
    if sparse:
        # the library's lists against the oracle's selection; the attention
        # then runs with the oracle's lists (neither half feeds the other)
        n_hist = len(s.frames) - wl.lat_t
        keep = sa.sparse_keep(n_hist * -(-wl.P // 64), sparse)
        it = s.item()
        it.n_hist_frames, it.keep_blocks = n_hist, keep
        got_lists = sa.sparse_select(s.geom, it).cpu().numpy()
        want_lists, scores = s.oracle_select(n_hist, keep)
        check_block_lists(got_lists, want_lists, scores, 1e-4 if wl.kv_dtype == "bf16" else 1e-3)
        s.set_sparse(want_lists, n_hist)
    sa.segment_attention(s.geom, [s.item()], workspace="auto" if split else None)
    torch.cuda.synchronize()
    got, got_lse = s.gpu_out()
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(got_lse)), label
    if wl.kv_dtype == "bf16":
        want, want_lse = s.oracle()
        _, _, rel = compare(got, want, 2e-2, 2e-3, label)
        assert rel <= 1e-2
        np.testing.assert_allclose(got_lse, want_lse, atol=4e-3, rtol=0)
    elif wl.kv_dtype == "int8":
        want, want_lse = s.oracle_int8_cache()
        _, _, rel = compare(got, want, 2e-2, 2e-3, label)
        assert rel <= 1e-2
        np.testing.assert_allclose(got_lse, want_lse, atol=5e-3, rtol=0)
    else:
        want, want_lse, bound = s.oracle_fp8_cache()
        err = np.abs(got - want)
        worst = float(np.max(err / (bound + 5e-3)))
        rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
        print(f"  max_abs={err.max():.3e} rel_l2={rel:.3e} max(err / (bound + 5e-3))={worst:.3f}",
              flush=True)
        assert worst <= 1.0 and rel <= 0.05
        np.testing.assert_allclose(got_lse, want_lse, atol=2e-2, rtol=0)
