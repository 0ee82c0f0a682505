"""GPU checks of history_gather (bit-exact byte copy of the picked frames) and
kv_dequant (e4m3 code times fp32 scale, rounded to bf16, against the oracle's
decode taken in the same fp32 precision).

Source planes are filled with random bytes by torch, not by the library, so
the expected values never come from the HIP path.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
from oracle import numerics

pytestmark = pytest.mark.gpu


def _fill_random(layer, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in (layer.k, layer.v, layer.k_text, layer.v_text):
        b = t.view(torch.uint8)
        b.copy_(torch.randint(0, 256, b.shape, generator=g, device="cuda", dtype=torch.uint8))
        if layer.dtype == sa.KV_FP8:
            b[(b & 0x7F) == 0x7F] = 0x3C           # keep codes finite
        elif layer.dtype == sa.KV_BF16:
            t.view(torch.int16)[torch.isnan(t.float())] = 0
    if layer.dtype in (sa.KV_FP8, sa.KV_INT8):
        for t in (layer.k_scale, layer.v_scale, layer.k_text_scale, layer.v_text_scale):
            t.copy_(torch.rand(t.shape, generator=g, device="cuda") * 0.05 + 0.001)


@pytest.mark.parametrize("dtype,grid", [(sa.KV_BF16, (4, 6)), (sa.KV_FP8, (4, 8)),
                                        (sa.KV_INT8, (4, 8)), (sa.KV_FP8, (4, 6)),
                                        (sa.KV_INT8, (4, 6)), (sa.KV_BF16, (22, 40)),
                                        (sa.KV_INT8, (22, 40))])
def test_gather_bit_exact(dtype, grid):
    H = 16 if grid == (22, 40) else 3
    geom = sa.Geom(heads=H, lat_h=grid[0], lat_w=grid[1])
    src = sa.KVLayer.allocate(geom, dtype, 40, 16)
    _fill_random(src, 1)
    frames = [39, 0, 17, 18, 5, 33]
    dst = sa.KVLayer.allocate(geom, dtype, len(frames) + 1, 16)
    d_frames = torch.tensor(frames, dtype=torch.int32, device="cuda")
    sa.history_gather(geom, src, d_frames, len(frames), dst)
    torch.cuda.synchronize()
    idx = torch.tensor(frames, device="cuda")
    assert torch.equal(dst.k[:len(frames)].view(torch.uint8), src.k[idx].view(torch.uint8))
    assert torch.equal(dst.v[:len(frames)].view(torch.uint8), src.v[idx].view(torch.uint8))
    if dtype != sa.KV_BF16:       # per plane (fp8) or per token (int8)
        assert torch.equal(dst.k_scale[:len(frames)], src.k_scale[idx])
        assert torch.equal(dst.v_scale[:len(frames)], src.v_scale[idx])


def _dequant_ref(codes, scale):
    """Oracle decode, product taken in fp32, then bf16 nearest-even (as bits)."""
    val = numerics.e4m3_decode(codes).astype(np.float32) * np.float32(scale)
    return numerics.bf16_bits(numerics.bf16_round(val.astype(np.float32).astype(np.float64)))


@pytest.mark.parametrize("n_text,lw", [(0, 8), (16, 8), (29, 8), (16, 6)])
def test_dequant_matches_oracle(n_text, lw):
    """e4m3 planes to bf16 planes; frames of 24 tokens come from planes of
    32 slots and go to planes of 24."""
    H = 3
    P = 4 * lw
    geom = sa.Geom(heads=H, lat_h=4, lat_w=lw)
    src = sa.KVLayer.allocate(geom, sa.KV_FP8, 10, 32)
    _fill_random(src, 2)
    frames = [9, 2, 4]
    dst = sa.KVLayer.allocate(geom, sa.KV_BF16, 3, 32)
    dst.k.zero_()
    dst.v.zero_()
    dst.k_text.zero_()
    dst.v_text.zero_()
    d_frames = torch.tensor(frames, dtype=torch.int32, device="cuda")
    sa.kv_dequant(geom, src, d_frames, len(frames), n_text, dst)
    torch.cuda.synchronize()
    sk, sv = src.k.cpu().numpy(), src.v.cpu().numpy()
    ks, vs = src.k_scale.cpu().numpy(), src.v_scale.cpu().numpy()
    gk = dst.k.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = dst.v.view(torch.int16).cpu().numpy().view(np.uint16)
    for i, f in enumerate(frames):
        for h in range(H):
            assert np.array_equal(gk[i, h], _dequant_ref(sk[f, h, :P], ks[f, h]))
            assert np.array_equal(gv[i, h], _dequant_ref(sv[f, h, :, :P], vs[f, h]))
    if n_text:
        tk = dst.k_text.view(torch.int16).cpu().numpy().view(np.uint16)
        tv = dst.v_text.view(torch.int16).cpu().numpy().view(np.uint16)
        sk, sv = src.k_text.cpu().numpy(), src.v_text.cpu().numpy()
        kts, vts = src.k_text_scale.cpu().numpy(), src.v_text_scale.cpu().numpy()
        for h in range(H):
            assert np.array_equal(tk[h, :n_text], _dequant_ref(sk[h, :n_text], kts[h]))
            assert np.array_equal(tv[h, :, :n_text], _dequant_ref(sv[h, :, :n_text], vts[h]))
            assert np.all(tk[h, n_text:] == 0) and np.all(tv[h, :, n_text:] == 0)


def _dequant_int8_ref(codes, scale):
    """code * scale in fp32, then bf16 nearest-even (as bits)."""
    val = codes.astype(np.float32) * scale.astype(np.float32)
    return numerics.bf16_bits(numerics.bf16_round(val.astype(np.float32).astype(np.float64)))


@pytest.mark.parametrize("n_text,lw", [(0, 8), (29, 8), (29, 6)])
def test_dequant_int8_matches_oracle(n_text, lw):
    """int8 planes with a scale per token and head: K rows scale per row, V^T
    columns per column; frames of 24 tokens come from planes of 32 slots."""
    H, lh = 3, 4
    P = lh * lw
    geom = sa.Geom(heads=H, lat_h=lh, lat_w=lw)
    src = sa.KVLayer.allocate(geom, sa.KV_INT8, 10, 32)
    _fill_random(src, 3)
    frames = [9, 2, 4]
    dst = sa.KVLayer.allocate(geom, sa.KV_BF16, 3, 32)
    for t in (dst.k, dst.v, dst.k_text, dst.v_text):
        t.zero_()
    d_frames = torch.tensor(frames, dtype=torch.int32, device="cuda")
    sa.kv_dequant(geom, src, d_frames, len(frames), n_text, dst)
    torch.cuda.synchronize()
    sk, sv = src.k.cpu().numpy(), src.v.cpu().numpy()
    ks, vs = src.k_scale.cpu().numpy(), src.v_scale.cpu().numpy()
    gk = dst.k.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = dst.v.view(torch.int16).cpu().numpy().view(np.uint16)
    for i, f in enumerate(frames):
        for h in range(H):
            assert np.array_equal(gk[i, h], _dequant_int8_ref(sk[f, h, :P], ks[f, h, :P][:, None]))
            assert np.array_equal(gv[i, h], _dequant_int8_ref(sv[f, h, :, :P], vs[f, h, :P][None, :]))
    if n_text:
        tk = dst.k_text.view(torch.int16).cpu().numpy().view(np.uint16)
        tv = dst.v_text.view(torch.int16).cpu().numpy().view(np.uint16)
        sk, sv = src.k_text.cpu().numpy(), src.v_text.cpu().numpy()
        kts, vts = src.k_text_scale.cpu().numpy(), src.v_text_scale.cpu().numpy()
        for h in range(H):
            assert np.array_equal(tk[h, :n_text], _dequant_int8_ref(sk[h, :n_text], kts[h, :n_text, None]))
            assert np.array_equal(tv[h, :, :n_text], _dequant_int8_ref(sv[h, :, :n_text], vts[h, None, :n_text]))


@pytest.mark.parametrize("src_kind", ["fp8", "int8"])
def test_dequant_into_uninitialised_layer_then_attend(src_kind):
    """kv_dequant into a bf16 layer whose planes hold NaN, then attention over
    the dequantised frames and n_text = 29 text keys (not a multiple of the
    64-key tile): the dequant writes zeros into the value plane's text columns
    [29, 32), so the attention meets finite values there and the output
    matches the oracle over the values the narrow cache stores (bf16 bar;
    the dequant's own bf16 rounding is far inside it)."""
    from helpers import Session
    import seeded_inputs as si
    wl = si.Workload(f"dq_{src_kind}", heads=2, lat_t=2, lat_h=4, lat_w=8, n_text=29,
                     prior_segments=(1,), kv_dtype=src_kind)
    s = Session(wl, seed=5, layer=0, session=0)
    n_frames = len(s.frames)
    assert s.frames == list(range(n_frames))           # slot i of dst holds frame i
    dst = sa.KVLayer.allocate(s.geom, sa.KV_BF16, n_frames, 32)
    nan = torch.tensor(0x7FC0, dtype=torch.int16).view(torch.bfloat16).item()
    for t in (dst.k, dst.v, dst.k_text, dst.v_text):
        t.fill_(nan)
    sa.kv_dequant(s.geom, s.kv, s.d_frames, n_frames, wl.n_text, dst)
    torch.cuda.synchronize()
    assert torch.all(dst.v_text[:, :, wl.n_text:] == 0)
    assert not torch.isnan(dst.v_text[:, :, :wl.n_text].float()).any()
    out = torch.empty_like(s.q)
    item = sa.AttnItem(s.q, dst, s.d_frames, n_frames, wl.n_text, out, frame0_q=s.S * wl.lat_t,
                       n_frames_q=wl.lat_t, n_text_q=wl.n_text)
    sa.segment_attention(s.geom, [item], workspace=None)
    torch.cuda.synchronize()
    got = out.float().cpu().double().numpy()
    assert np.all(np.isfinite(got))
    if src_kind == "fp8":
        want, _, _ = s.oracle_fp8_cache()
    else:
        want, _ = s.oracle_int8_cache()
    err = np.abs(got - want)
    print(f"dequant {src_kind} then attend: max_abs={err.max():.3e} mean_abs={err.mean():.3e}",
          flush=True)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
