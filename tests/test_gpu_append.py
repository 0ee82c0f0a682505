"""GPU parity of kv_append / text_append against the oracle (through the C ABI).

Gates: V planes bit-exact (a pure transposed copy); K planes: at least 99.9 %
of elements bit-identical to the oracle's exactly rotated, correctly rounded
keys, and every element within one bf16 ulp of the exact rotation plus the
fp32 rotation error, 1e-6 times the magnitude of the rotated pair (a rotated
value near zero is the difference of two products, so its own ulp is no
bound); K at position (0, 0, 0) bit-exact; frames outside the written range
untouched. fp8: V codes and all scales follow the fp32 decision
exactly; K codes within one code step.
"""

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
import seeded_inputs as si
from oracle import cache as ocache
from oracle import numerics
from oracle import rope as orope
from e4m3_cases import TIE_CODES, TIE_VALUES

pytestmark = pytest.mark.gpu

SPLIT = (16, 56, 56)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _ordered(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _ulp_diff(a_bits, b_bits):
    return np.abs(_ordered(a_bits) - _ordered(b_bits))


@pytest.mark.parametrize("shape", [(3, 4, 6, 3, 5, 10000.0), (2, 4, 8, 2, 0, 256.0),
                                   (16, 22, 40, 30, 30, 10000.0)])
def test_kv_append_bf16(shape):
    H, lh, lw, F, frame0, theta = shape
    print(f"kv_append bf16 H={H} grid={lh}x{lw} F={F} frame0={frame0}", flush=True)
    P = lh * lw
    geom = sa.Geom(heads=H, lat_h=lh, lat_w=lw, rope_theta=theta)
    cap = frame0 + F + 2
    layer = sa.KVLayer.allocate(geom, sa.KV_BF16, cap, 16)
    sentinel = torch.tensor(0x7FC0, dtype=torch.int16).view(torch.bfloat16)   # bf16 NaN
    layer.k.fill_(sentinel.item())
    layer.v.fill_(sentinel.item())
    k = si.normal_bf16((F * P, H, 128), 11, "cuda")
    v = si.normal_bf16((F * P, H, 128), 12, "cuda")
    sa.kv_append(geom, layer, k, v, frame0, F)
    torch.cuda.synchronize()
    K, V = ocache.append_bf16(k.float().cpu().double().numpy(), v.float().cpu().double().numpy(),
                              frame0, lh, lw, SPLIT, theta)
    gotV = _bits(layer.v[frame0:frame0 + F])
    assert np.array_equal(gotV, numerics.bf16_bits(V))
    gotK = _bits(layer.k[frame0:frame0 + F])
    wantK = numerics.bf16_bits(K)
    ulp = _ulp_diff(gotK, wantK)
    frac = float(np.mean(ulp == 0))
    print(f"  K bitwise fraction {frac:.6f}, max ulp {ulp.max()}", flush=True)
    assert frac >= 0.999
    kin = k.float().cpu().double().numpy()
    exact = orope.rope3d(kin, orope.video_positions(frame0, F, lh, lw), SPLIT, theta)
    exact = exact.reshape(F, P, H, 128).transpose(0, 2, 1, 3)
    pair = np.sqrt(exact[..., 0::2] ** 2 + exact[..., 1::2] ** 2).repeat(2, axis=-1)
    _, e = np.frexp(np.maximum(np.abs(exact), 2.0 ** -126))
    ulp_exact = np.ldexp(1.0, e - 1 - 7)
    err = np.abs(numerics.bf16_from_bits(gotK) - exact)
    assert np.all(err <= ulp_exact + 1e-6 * pair)
    if frame0 == 0:
        assert np.array_equal(gotK[0, :, 0, :], _bits(k[0]))
    untouched = torch.cat([layer.k[:frame0].flatten(), layer.k[frame0 + F:].flatten()])
    assert torch.isnan(untouched.float()).all()
    untouched = torch.cat([layer.v[:frame0].flatten(), layer.v[frame0 + F:].flatten()])
    assert torch.isnan(untouched.float()).all()


@pytest.mark.parametrize("n_text,cap", [(16, 16), (37, 48), (256, 256), (0, 16)])
def test_text_append_bf16(n_text, cap):
    H = 3
    geom = sa.Geom(heads=H, lat_h=4, lat_w=6)
    layer = sa.KVLayer.allocate(geom, sa.KV_BF16, 1, cap)
    layer.v_text.fill_(float("nan"))
    k = si.normal_bf16((max(n_text, 1), H, 128), 21, "cuda")
    v = si.normal_bf16((max(n_text, 1), H, 128), 22, "cuda")
    sa.text_append(geom, layer, k, v, n_text)
    torch.cuda.synchronize()
    if n_text:
        assert torch.equal(layer.k_text[:, :n_text].view(torch.int16),
                           k[:n_text].transpose(0, 1).contiguous().view(torch.int16))
        assert torch.equal(layer.v_text[:, :, :n_text].view(torch.int16),
                           v[:n_text].permute(1, 2, 0).contiguous().view(torch.int16))
    # value columns past n_text are zeroed (finite for masked key chunks)
    assert torch.all(layer.v_text[:, :, n_text:] == 0)


@pytest.mark.parametrize("shape", [(2, 4, 8, 3, 2), (2, 4, 6, 3, 1), (16, 22, 40, 2, 7)])
def test_kv_append_fp8(shape):
    """Frames of 24 tokens fill planes of 32 slots: the V^T tail holds zero
    codes."""
    H, lh, lw, F, frame0 = shape
    print(f"kv_append fp8 H={H} grid={lh}x{lw} F={F}", flush=True)
    P = lh * lw
    geom = sa.Geom(heads=H, lat_h=lh, lat_w=lw)
    layer = sa.KVLayer.allocate(geom, sa.KV_FP8, frame0 + F, 16)
    assert layer.v.shape[-1] == ocache.plane_slots("fp8", P)
    layer.v.fill_(0x5A)
    wl = si.Workload("t", heads=H, lat_t=F, lat_h=lh, lat_w=lw, n_text=16, prior_segments=(0,),
                     kv_dtype="fp8", scale_factors=True)
    k, v = si.segment_kv(wl, 3, 0, 0, 0, "cuda")
    sa.kv_append(geom, layer, k, v, frame0, F)
    torch.cuda.synchronize()
    Kc, Ks, Vc, Vs = ocache.append_fp8(k.float().cpu().double().numpy(),
                                       v.float().cpu().double().numpy(), frame0, lh, lw, SPLIT, 10000.0)
    gotVc = layer.v[frame0:].cpu().numpy()
    gotVs = layer.v_scale[frame0:].cpu().numpy()
    assert np.array_equal(gotVs, Vs)
    assert np.array_equal(gotVc[..., :P], Vc)
    assert np.all(gotVc[..., P:] == 0)
    gotKs = layer.k_scale[frame0:].cpu().numpy()
    np.testing.assert_allclose(gotKs, Ks, rtol=2e-6)
    gotKc = layer.k[frame0:, :, :P].cpu().numpy()
    step = np.abs(_e4m3_ordered(gotKc) - _e4m3_ordered(Kc))
    print(f"  K code agreement {np.mean(step == 0):.6f}", flush=True)
    assert step.max() <= 1
    assert np.mean(step == 0) >= 0.99


def _e4m3_ordered(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def test_text_append_fp8():
    H, n = 4, 40
    geom = sa.Geom(heads=H, lat_h=4, lat_w=8)
    layer = sa.KVLayer.allocate(geom, sa.KV_FP8, 1, 48)
    k = si.normal_bf16((n, H, 128), 31, "cuda")
    v = si.normal_bf16((n, H, 128), 32, "cuda")
    sa.text_append(geom, layer, k, v, n)
    torch.cuda.synchronize()
    Kc, Ks, Vc, Vs = ocache.append_text_fp8(k.float().cpu().double().numpy(),
                                            v.float().cpu().double().numpy())
    assert np.array_equal(layer.k_text_scale.cpu().numpy(), Ks)
    assert np.array_equal(layer.v_text_scale.cpu().numpy(), Vs)
    assert np.array_equal(layer.k_text[:, :n].cpu().numpy(), Kc)
    assert np.array_equal(layer.v_text[:, :, :n].cpu().numpy(), Vc)
    assert np.all(layer.v_text[:, :, n:].cpu().numpy() == 0)


# ------------------------------------------------------------------- int8 cache
@pytest.mark.parametrize("shape", [(2, 4, 8, 3, 2), (2, 4, 6, 3, 1), (16, 22, 40, 2, 7)])
def test_kv_append_int8(shape):
    """int8 with a scale per token and head: V codes and scales bit-exact
    (fp32 decisions on both sides); K is rotated in fp32 by the kernel and in
    exact arithmetic by the oracle, so a K code may move one step near a
    rounding boundary and a K scale by fp32 rounding. Frames of 24 tokens
    fill planes of 32 slots: zero V^T codes and zero scales in the tail."""
    H, lh, lw, F, frame0 = shape
    print(f"kv_append int8 H={H} grid={lh}x{lw} F={F}", flush=True)
    P = lh * lw
    geom = sa.Geom(heads=H, lat_h=lh, lat_w=lw)
    layer = sa.KVLayer.allocate(geom, sa.KV_INT8, frame0 + F, 16)
    layer.v.fill_(0x5A)
    layer.k_scale.fill_(float("nan"))
    layer.v_scale.fill_(float("nan"))
    wl = si.Workload("t", heads=H, lat_t=F, lat_h=lh, lat_w=lw, n_text=16, prior_segments=(0,),
                     kv_dtype="fp8", scale_factors=True)
    k, v = si.segment_kv(wl, 5, 0, 0, 0, "cuda")
    sa.kv_append(geom, layer, k, v, frame0, F)
    torch.cuda.synchronize()
    Kc, Ks, Vc, Vs = ocache.append_int8(k.float().cpu().double().numpy(),
                                        v.float().cpu().double().numpy(), frame0, lh, lw, SPLIT, 10000.0)
    assert np.array_equal(layer.v_scale[frame0:, :, :P].cpu().numpy(), Vs)
    assert np.array_equal(layer.v[frame0:, :, :, :P].cpu().numpy(), Vc)
    assert np.all(layer.v[frame0:, :, :, P:].cpu().numpy() == 0)
    assert np.all(layer.k_scale[frame0:, :, P:].cpu().numpy() == 0)
    assert np.all(layer.v_scale[frame0:, :, P:].cpu().numpy() == 0)
    np.testing.assert_allclose(layer.k_scale[frame0:, :, :P].cpu().numpy(), Ks, rtol=2e-6)
    step = np.abs(layer.k[frame0:, :, :P].cpu().numpy().astype(np.int32) - Kc.astype(np.int32))
    print(f"  K code agreement {np.mean(step == 0):.6f}", flush=True)
    assert step.max() <= 1
    assert np.mean(step == 0) >= 0.99


def test_text_append_int8():
    H, n = 4, 40
    geom = sa.Geom(heads=H, lat_h=4, lat_w=8)
    layer = sa.KVLayer.allocate(geom, sa.KV_INT8, 1, 48)
    layer.k_text_scale.fill_(float("nan"))
    layer.v_text_scale.fill_(float("nan"))
    k = si.normal_bf16((n, H, 128), 33, "cuda")
    v = si.normal_bf16((n, H, 128), 34, "cuda")
    sa.text_append(geom, layer, k, v, n)
    torch.cuda.synchronize()
    Kc, Ks, Vc, Vs = ocache.append_text_int8(k.float().cpu().double().numpy(),
                                             v.float().cpu().double().numpy())
    assert np.array_equal(layer.k_text_scale[:, :n].cpu().numpy(), Ks)
    assert np.array_equal(layer.v_text_scale[:, :n].cpu().numpy(), Vs)
    assert np.array_equal(layer.k_text[:, :n].cpu().numpy(), Kc)
    assert np.array_equal(layer.v_text[:, :, :n].cpu().numpy(), Vc)
    # tokens past n_text: zero codes in V and zero scales (finite for masked keys)
    assert np.all(layer.v_text[:, :, n:].cpu().numpy() == 0)
    assert np.all(layer.k_text_scale[:, n:].cpu().numpy() == 0)
    assert np.all(layer.v_text_scale[:, n:].cpu().numpy() == 0)


def test_text_append_fp8_ties_and_subnormals():
    """A text slot whose largest magnitude is 448, so the scale is exactly 1 and
    the stored codes are the e4m3 roundings of the inputs themselves: exact
    ties between neighbouring codes (normal and subnormal, resolved to the even
    code), the largest code, and values that round up into the normal range."""
    H, n = 2, 16
    ties = TIE_VALUES
    x = np.resize(np.array(ties, dtype=np.float32), (n, H, 128))
    g = np.random.default_rng(7)
    mix = g.random(x.shape) < 0.5
    mix[0] = False                           # token 0 keeps the listed values
    x = np.where(mix, np.float32(g.standard_normal(x.shape) * 4), x)
    k = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(k.float().numpy()[0], x[0])     # the listed values are bf16-exact
    assert np.all(np.abs(k.float().numpy()).max(axis=(0, 2)) == 448.0)
    kd = k.cuda()
    geom = sa.Geom(heads=H, lat_h=4, lat_w=8)
    layer = sa.KVLayer.allocate(geom, sa.KV_FP8, 1, 16)
    sa.text_append(geom, layer, kd, kd, n)
    torch.cuda.synchronize()
    xd = k.float().double().numpy()
    Kc, Ks, Vc, Vs = ocache.append_text_fp8(xd, xd)
    assert np.all(Ks == 1.0) and np.all(Vs == 1.0)
    assert np.array_equal(layer.k_text_scale.cpu().numpy(), Ks)
    assert np.array_equal(layer.k_text[:, :n].cpu().numpy(), Kc)
    assert np.array_equal(layer.v_text[:, :, :n].cpu().numpy(), Vc)
    # the ties themselves went to the even code
    codes = layer.k_text[0, 0, :len(ties)].cpu().numpy()
    print("tie codes", [hex(c) for c in codes], flush=True)
    assert np.array_equal(codes, TIE_CODES)
