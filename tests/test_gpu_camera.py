"""GPU parity of camera cross-attention against the oracle (oracle/camera.py).

The video tokens of latent frame t attend to the camera tokens of their chunk
(chunk 1: only their own; "Hy-Nomas: an 8.6B world model ...", section "The
camera"). Closed form: with chunk 1 each output row is its frame's camera
value bit for bit and lse is the scaled q.k. Other chunks, shared and
per-head camera keys, ragged last chunks and extra camera tokens are checked
against the oracle (bf16 inputs are exact, so the bar is fp32 arithmetic plus
the bf16 output rounding: max-abs 1e-2, mean-abs 1e-3, relative L2 4e-3).
"""

import math

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import compare
from oracle import camera as ocam

pytestmark = pytest.mark.gpu


def _inputs(F, lh, lw, H, n_cam, hk, seed):
    geom = sa.Geom(heads=H, lat_h=lh, lat_w=lw)
    P = lh * lw
    q = si.normal_bf16((F * P, H, 128), si.derive_seed(seed, "camera", "q"), "cuda")
    ck = si.normal_bf16((n_cam, hk, 128), si.derive_seed(seed, "camera", "k"), "cuda")
    cv = si.normal_bf16((n_cam, hk, 128), si.derive_seed(seed, "camera", "v"), "cuda")
    return geom, P, q, ck, cv


def _run(geom, F, q, ck, cv, chunk):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    sa.camera_attention(geom, q, F, ck, cv, chunk, out, lse)
    torch.cuda.synchronize()
    return out, lse


def _np(t):
    return t.float().cpu().double().numpy()


@pytest.mark.parametrize("hk", [1, 3])
def test_chunk_one_copies_camera_value(hk):
    F, H = 5, 3
    geom, P, q, ck, cv = _inputs(F, 4, 6, H, F, hk, 1)
    out, lse = _run(geom, F, q, ck, cv, 1)
    o = out.view(torch.int16).cpu().numpy()
    v = cv.view(torch.int16).cpu().numpy()
    for t in range(F):
        want = v[t, [0] * H if hk == 1 else list(range(H))]
        assert np.array_equal(o[t * P:(t + 1) * P], np.broadcast_to(want, (P, H, 128)))
    wq, wk = _np(q), _np(ck)
    t = np.arange(F * P) // P
    hs = np.zeros(H, int) if hk == 1 else np.arange(H)
    want_lse = np.einsum("rhd,rhd->rh", wq, wk[t][:, hs]) / math.sqrt(128)
    np.testing.assert_allclose(lse.cpu().numpy(), want_lse, atol=1e-4, rtol=1e-5)


CASES = [
    # F, lat_h, lat_w, H, n_cam, kv_heads, chunk
    (6, 4, 6, 2, 6, 1, 2),
    (7, 4, 6, 2, 7, 2, 3),      # ragged last chunk (frame 6 alone)
    (5, 8, 10, 4, 8, 1, 4),     # extra camera tokens: frame 4's chunk is tokens 4..7
    (4, 4, 8, 2, 4, 2, 16),     # one chunk over every token
    (9, 4, 4, 3, 9, 3, 16),     # the largest chunk
]


@pytest.mark.parametrize("case", CASES, ids=[f"F{c[0]}-hk{c[5]}-c{c[6]}" for c in CASES])
def test_chunks_match_oracle(case):
    F, lh, lw, H, n_cam, hk, chunk = case
    print(f"camera attention case={case}", flush=True)
    geom, P, q, ck, cv = _inputs(F, lh, lw, H, n_cam, hk, 2)
    out, lse = _run(geom, F, q, ck, cv, chunk)
    want, want_lse = ocam.camera_attention(_np(q), _np(ck), _np(cv), P, chunk)
    got = _np(out)
    _, _, rel = compare(got, want, 1e-2, 1e-3, str(case))
    assert rel <= 4e-3
    np.testing.assert_allclose(lse.cpu().numpy(), want_lse, atol=1e-4, rtol=1e-5)


def test_full_segment():
    """The pages' segment: 30 latent frames of 22 x 40 tokens, 16 heads, one
    shared camera head. Chunk 1 over every row (closed form), chunk 4 on
    sampled rows against the oracle."""
    F, H = 30, 16
    geom, P, q, ck, cv = _inputs(F, 22, 40, H, F, 1, 3)
    out, _ = _run(geom, F, q, ck, cv, 1)
    o = out.view(torch.int16).cpu().numpy()
    v = cv.view(torch.int16).cpu().numpy()
    for t in range(F):
        assert np.array_equal(o[t * P:(t + 1) * P], np.broadcast_to(v[t, [0] * H], (P, H, 128)))
    out, lse = _run(geom, F, q, ck, cv, 4)
    rows = si.sample_rows(F * P, 256, 5, [P - 1, P, 4 * P - 1, 4 * P, 28 * P])
    want, want_lse = ocam.camera_attention(_np(q), _np(ck), _np(cv), P, 4)
    got = _np(out)[rows]
    _, _, rel = compare(got, want[rows], 1e-2, 1e-3, "full segment chunk 4")
    assert rel <= 4e-3
    np.testing.assert_allclose(lse.cpu().numpy()[rows], want_lse[rows], atol=1e-4, rtol=1e-5)
