"""sa_segment_attention_counted: the same outputs as sa_segment_attention, bit
for bit, plus counts of the softmax's rescaling paths.

On N(0, 1) inputs at the 1/sqrt(128) scale attention is near-uniform and the
slow paths do not run; with the queries scaled by 40, rows meet keys hundreds
of log2 units above their first block's max (tests/test_gpu_attention.py
checks that such rises exist for these seeds and shapes), so the bf16 kernel
re-runs work tiles with rescaling and the e4m3 kernel renormalises.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from helpers import Session

pytestmark = pytest.mark.gpu


def _wl(kv):
    if kv == "bf16":
        return si.Workload("cnt_bf16", heads=2, lat_t=4, lat_h=6, lat_w=8, n_text=24,
                           prior_segments=(2,))
    return si.Workload("cnt_fp8", heads=2, lat_t=4, lat_h=6, lat_w=8, n_text=24,
                       prior_segments=(8,), kv_dtype="fp8", scale_factors=True)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("q_scale", [1.0, 40.0])
def test_counted_attention(kv, q_scale):
    wl = _wl(kv)
    print(f"counted attention {kv} q*{q_scale}", flush=True)
    s = Session(wl, seed=13, layer=0, session=0, q_scale=q_scale)
    sa.segment_attention(s.geom, [s.item()], workspace=None)
    torch.cuda.synchronize()
    want, want_lse = s.out.clone(), s.lse.clone()
    s.out.zero_()
    c = torch.zeros(3, dtype=torch.int32, device="cuda")
    sa.segment_attention(s.geom, [s.item()], workspace=None, counters=c)
    torch.cuda.synchronize()
    assert torch.equal(s.out.view(torch.int16), want.view(torch.int16))
    assert torch.equal(s.lse.view(torch.int32), want_lse.view(torch.int32))
    tiles, slow, resc = (int(x) for x in c.cpu())
    print(f"{kv} q*{q_scale}: work tiles {tiles}, slow-path events {slow}, rescale steps {resc}",
          flush=True)
    assert tiles == wl.heads * -(-wl.Lq // 256)
    if q_scale == 1.0:
        assert slow == 0
    else:
        assert slow > 0 and resc > 0
    # counts add up over calls; with the split workspace there are more work tiles
    sa.segment_attention(s.geom, [s.item()], counters=c)
    torch.cuda.synchronize()
    assert int(c[0]) >= 2 * tiles
    assert np.isfinite(s.out.float().cpu().numpy()).all()
