"""Pins for oracle.cache (byte counts, plane layout, expected append contents).

Byte counts are pinned by the figures printed on the page ("Hy-Nomas: an 8.6B
world model ...", sections "What 'world memory' stores" and "The 4090 preset",
stored in tests/golden/page_figures.json). Layout maps are pinned by brute
force (bijection onto the plane; agreement with numpy's own transposes).
Append contents are pinned by exact cases (V is a copy; position (0,0,0) is the
identity rotation) and by the explicit per-row rotation.
"""

import json
import os

import numpy as np

from oracle import cache, numerics, rope
from e4m3_cases import TIE_CODES, TIE_VALUES, nearest_code_brute

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_token_grid_figures():
    g = FIG["token_grid"]
    assert g["frame_h_px"] // g["spatial_factor"] == g["lat_h"]
    assert g["frame_w_px"] // g["spatial_factor"] == g["lat_w"]
    assert g["lat_h"] * g["lat_w"] == g["tokens_per_frame"]
    assert g["tokens_per_frame"] * g["latent_frames_per_segment"] == g["tokens_per_segment"]
    assert g["heads"] * g["head_dim"] == g["hidden"]
    assert sum(g["rope_split"]) == g["head_dim"]


def test_bf16_bytes_match_page():
    f = FIG["bf16_cache"]
    g = FIG["token_grid"]
    b = cache.bytes_per_token_per_layer("bf16", g["heads"], g["head_dim"])
    assert b == f["bytes_per_token_per_layer"]
    assert b * g["layers"] == f["bytes_per_token_54_layers"]
    per_frame = b * g["layers"] * g["tokens_per_frame"]
    assert round(per_frame / 1e6) == f["mb_per_frame"]
    per_s = per_frame * f["latent_fps"]
    assert round(per_s / 1e9, 2) == f["gb_per_second"]
    assert round(per_s * 60 / 1e9) == f["gb_per_minute"]
    assert round(per_s * 60 / 8 / 1e9, 1) == f["gb_per_gpu_sp8"]


def test_int8_bytes_match_page():
    f = FIG["int8_cache"]
    g = FIG["token_grid"]
    b = cache.bytes_per_token_per_layer("int8_token_head", g["heads"], g["head_dim"])
    assert b == f["bytes_per_token_per_layer"]
    per_frame = b * g["layers"] * g["tokens_per_frame"]
    assert round(per_frame * f["kept_frames"] / 1e9, 1) == f["gb_kept"]
    assert round(per_frame / 1e6, -2) == f["mb_per_frame"]
    assert round(per_frame * 6 / 1e9, 1) == f["gb_per_second"]
    assert round(per_frame * 6 * 60 / 1e9) == f["gb_per_minute"]


def test_plane_bytes():
    assert cache.plane_bytes("bf16", 16, 128, 880, 60, 256) == 2 * 2 * 2048 * (60 * 880 + 256)
    assert cache.plane_bytes("fp8", 16, 128, 880, 60, 256) == 2 * 2048 * (60 * 880 + 256) + 8 * 16 * 61


def test_padded_plane_slots_hand_worked():
    """One-byte caches pad a frame plane to a multiple of 16 token slots (so
    V^T rows start 16-byte aligned); bf16 planes keep P."""
    assert [cache.plane_slots("fp8", P) for P in (24, 136, 880, 16, 8)] == [32, 144, 880, 16, 16]
    assert cache.plane_slots("int8", 24) == 32 and cache.plane_slots("bf16", 24) == 24
    # H = 2, D = 128, P = 24 (32 slots), 3 frames, 16 text slots, worked by hand:
    # values 2 * 2 * 128 * (3 * 32 + 16) = 57,344 bytes
    assert cache.plane_bytes("fp8", 2, 128, 24, 3, 16) == 57_344 + 2 * 4 * 2 * 4
    assert cache.plane_bytes("int8", 2, 128, 24, 3, 16) == 57_344 + 2 * 4 * 2 * (96 + 16)
    assert cache.plane_bytes("bf16", 2, 128, 24, 3, 16) == 2 * 2 * 2 * 128 * (72 + 16)


def test_padded_layout_leaves_exactly_the_tail_slots_unused():
    F, H, P, PL, D = 2, 3, 6, 16, 4
    ko = {cache.k_offset(f, h, p, c, H, PL, D) for f in range(F) for h in range(H)
          for p in range(P) for c in range(D)}
    vo = {cache.v_offset(f, h, p, c, H, PL, D) for f in range(F) for h in range(H)
          for p in range(P) for c in range(D)}
    assert len(ko) == len(vo) == F * H * P * D
    assert ko == {((f * H + h) * PL + p) * D + c for f in range(F) for h in range(H)
                  for p in range(P) for c in range(D)}
    unused_v = set(range(F * H * PL * D)) - vo
    assert unused_v == {((f * H + h) * D + c) * PL + p for f in range(F) for h in range(H)
                        for c in range(D) for p in range(P, PL)}


def test_layout_is_bijection_and_matches_numpy_transposes():
    F, H, P, D, TC = 3, 2, 6, 4, 5
    n = F * H * P * D
    ko = np.array([cache.k_offset(f, h, p, c, H, P, D) for f in range(F) for h in range(H)
                   for p in range(P) for c in range(D)])
    vo = np.array([cache.v_offset(f, h, p, c, H, P, D) for f in range(F) for h in range(H)
                   for p in range(P) for c in range(D)])
    assert sorted(ko.tolist()) == list(range(n)) and sorted(vo.tolist()) == list(range(n))
    x = np.arange(n).reshape(F, H, P, D)              # value = k-plane offset
    flatK = np.empty(n, dtype=np.int64)
    flatK[ko] = x.reshape(-1)
    assert np.array_equal(flatK, x.reshape(-1))
    flatV = np.empty(n, dtype=np.int64)
    flatV[vo] = x.reshape(-1)
    assert np.array_equal(flatV, x.transpose(0, 1, 3, 2).reshape(-1))
    tk = [cache.text_k_offset(h, i, c, TC, D) for h in range(H) for i in range(TC) for c in range(D)]
    tv = [cache.text_v_offset(h, i, c, TC, D) for h in range(H) for i in range(TC) for c in range(D)]
    assert sorted(tk) == list(range(H * TC * D)) and sorted(tv) == list(range(H * TC * D))


def _bf16_inputs(shape, seed):
    return numerics.bf16_round(np.random.default_rng(seed).standard_normal(shape))


def test_append_bf16_v_copy_and_k_rotation():
    lat_h, lat_w, H, D, F = 4, 6, 2, 128, 2
    P = lat_h * lat_w
    k = _bf16_inputs((F * P, H, D), 0)
    v = _bf16_inputs((F * P, H, D), 1)
    for frame0 in (0, 7):
        K, V = cache.append_bf16(k, v, frame0, lat_h, lat_w, (16, 56, 56), 10000.0)
        assert K.shape == (F, H, P, D) and V.shape == (F, H, D, P)
        for f in range(F):
            for p in range(P):
                tok = f * P + p
                assert np.array_equal(V[f, :, :, p], v[tok])
                pos = np.array([[frame0 + f, p // lat_w, p % lat_w]])
                want = numerics.bf16_round(rope.rope3d(k[tok], pos))
                assert np.array_equal(K[f, :, p, :], want)
        if frame0 == 0:
            assert np.array_equal(K[0, :, 0, :], k[0])          # position (0,0,0)


def test_append_text_is_identity_layout():
    k = _bf16_inputs((9, 3, 128), 2)
    v = _bf16_inputs((9, 3, 128), 3)
    K, V = cache.append_text_bf16(k, v)
    assert np.array_equal(K, k.transpose(1, 0, 2)) and np.array_equal(V, v.transpose(1, 2, 0))


def test_plane_scale_exponent_hand_worked():
    """The plane scale is the least power of two 2**e with amax <= 448 * 2**e:
    worked by hand at and around the boundaries (448 = 1.75 * 2**8)."""
    f32 = np.float32
    cases = [(448.0, 0), (np.nextafter(f32(448.0), f32(1e9)), 1), (224.0, -1),
             (np.nextafter(f32(224.0), f32(1e9)), 0), (1.0, -8), (1.75, -8),
             (np.nextafter(f32(1.75), f32(9.0)), -7), (3.0e38, 120), (1e-40, -126), (0.0, 0),
             (2.0 ** -120, -126), (448.0 * 2.0 ** -126, -126), (448.0 * 2.0 ** -125, -125)]
    for amax, e in cases:
        assert cache.plane_scale_exponent(f32(amax)) == e, (amax, e)


def test_quantize_plane_fp8_properties():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((24, 128)) * 1.7).astype(np.float32).astype(np.float64)
    codes, scale = cache.quantize_plane_fp8(x)
    amax = np.float32(np.abs(x).max())
    e = int(np.log2(scale))
    assert scale == 2.0 ** e                                # a power of two
    assert 224.0 < amax / scale <= 448.0                    # the least one that holds amax
    dq = cache.dequant(codes, scale)
    # relative error of e4m3 (3 mantissa bits) is at most 2**-4 for normals
    normal = np.abs(x) / scale >= 2.0 ** -6
    assert np.all(np.abs(dq - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 * 1.0001)
    assert np.all(np.abs(dq - x)[~normal] <= 2.0 ** -10 * scale * 1.0001)
    z, s0 = cache.quantize_plane_fp8(np.zeros((3, 4)))
    assert s0 == 1.0 and not z.any()


def _fp32_plane_codes(x):
    """Expected codes and scale of one plane from the reading of the format,
    by search rather than the oracle's own steps: the scale is the first power
    of two 2**e (e counted up from -126) with amax <= 448 * 2**e, and the codes
    are the nearest e4m3 codes of x / 2**e by exhaustive search."""
    x32 = np.asarray(x, dtype=np.float32).astype(np.float64)
    amax = np.abs(x32).max()
    e = -126
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return nearest_code_brute(x32 * 2.0 ** -e, numerics.e4m3_decode), np.float32(2.0 ** e)


def test_append_fp8_codes_are_brute_force_nearest_per_plane():
    """V codes of every (frame, head) plane are the nearest e4m3 codes of
    v * 448 / amax(plane), found by exhaustive search; every plane gets its
    own scale (each (frame, head) is scaled by its own factor here, so a
    scale shared across frames or heads fails); V is transposed per plane
    (V^T[d][p] holds token p's dim d); K codes are those of the rotated keys
    under the K plane's own scale."""
    lat_h, lat_w, H, F = 4, 6, 3, 2
    P = lat_h * lat_w
    # [F, H]; factors 4x apart, so that every plane's power-of-two scale differs
    fac = np.array([[1 / 16, 1.0, 1 / 4], [16.0, 1 / 64, 4.0]])
    k = _bf16_inputs((F * P, H, 128), 5) * np.repeat(fac, P, axis=0)[:, :, None]
    v = numerics.bf16_round(_bf16_inputs((F * P, H, 128), 6) * np.repeat(fac[::-1], P, axis=0)[:, :, None])
    Kc, Ks, Vc, Vs = cache.append_fp8(k, v, 3, lat_h, lat_w, (16, 56, 56), 10000.0)
    assert Kc.shape == (F, H, P, 128) and Vc.shape == (F, H, 128, P)
    assert Ks.shape == (F, H) and Vs.shape == (F, H)
    kr = rope.rope3d(k, rope.video_positions(3, F, lat_h, lat_w))
    for f in range(F):
        for h in range(H):
            vplane = v[f * P:(f + 1) * P, h, :]                        # [P, D]
            want, scale = _fp32_plane_codes(vplane)
            assert Vs[f, h] == scale
            assert np.array_equal(Vc[f, h], want.T)
            kplane = kr[f * P:(f + 1) * P, h, :]
            want_k, kscale = _fp32_plane_codes(kplane.astype(np.float32))
            assert Ks[f, h] == kscale
            assert np.array_equal(Kc[f, h], want_k)
    assert len(set(Vs.reshape(-1).tolist())) == F * H       # one scale per plane


def test_append_text_fp8_scale_per_head_and_hand_worked_codes():
    """The text slot: one scale per head over all of its tokens, no rotation,
    V transposed to [H][D][n]. Head 0 holds the hand-worked tie values in
    token 0 and smaller values elsewhere, so its amax is 448 and its scale
    exactly 1: token 0's codes are the hand-worked ones, and the other
    tokens' codes are the plain e4m3 roundings of their values (a per-token
    scale would stretch them). Head 1 is head 0 halved: scale exactly 0.5 and
    the same codes (a scale shared by the heads would give other codes)."""
    n, H = 12, 2
    rng = np.random.default_rng(9)
    base = numerics.bf16_round(rng.standard_normal((n, 128)) * 40.0)
    base = np.clip(base, -400.0, 400.0)
    base[0] = np.resize(np.array(TIE_VALUES), 128)
    x = np.stack([base, base * 0.5], axis=1)                      # [n, H, D]
    vx = x[:, :, ::-1].copy()                                     # V differs from K
    Kc, Ks, Vc, Vs = cache.append_text_fp8(x, vx)
    assert Kc.shape == (H, n, 128) and Vc.shape == (H, 128, n)
    assert Ks.tolist() == [1.0, 0.5] and Vs.tolist() == [1.0, 0.5]
    assert np.array_equal(Kc[0, 0, :16], TIE_CODES)
    assert np.array_equal(Kc[1], Kc[0])
    assert np.array_equal(Kc[0], nearest_code_brute(base, numerics.e4m3_decode))
    # V^T[h][d][i] holds token i's dim d; token 0 of V holds the ties reversed
    assert np.array_equal(Vc[0, 127 - np.arange(16), 0], TIE_CODES)
    assert np.array_equal(Vc[0], nearest_code_brute(base[:, ::-1], numerics.e4m3_decode).T)
    assert np.array_equal(Vc[1], Vc[0])
    # the hand-worked codes are also those of exhaustive search
    assert np.array_equal(nearest_code_brute(np.array(TIE_VALUES), numerics.e4m3_decode),
                          TIE_CODES)


# ------------------------------------------------------------------- int8 cache
def test_int8_plane_bytes_per_token_match_page():
    """The library's int8 layout spends exactly the page's 4,224 bytes per
    token per layer on frames (one byte per value, an fp32 scale per token
    and head, for K and V)."""
    g = FIG["token_grid"]
    H, D, P = g["heads"], g["head_dim"], g["tokens_per_frame"]
    one = cache.plane_bytes("int8", H, D, P, 1, 0)
    assert one == P * FIG["int8_cache"]["bytes_per_token_per_layer"]
    assert cache.plane_bytes("int8", H, D, P, 3, 32) == (3 * P + 32) * 4224


def _rng(seed):
    return np.random.default_rng(seed)


def test_int8_quantize_closed_forms():
    x = _rng(1).standard_normal((50, 128)).astype(np.float32) * 3
    codes, scale = cache.quantize_token_int8(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert codes.min() >= -127 and codes.max() <= 127
    # the largest magnitude of every vector maps to +-127
    i = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(50), i]) == 127)
    assert np.all(np.sign(codes[np.arange(50), i]) == np.sign(x[np.arange(50), i]))
    # scale is amax / 127
    np.testing.assert_allclose(scale, np.abs(x).max(axis=1) / 127.0, rtol=1e-7)
    # a zero vector: scale 1, codes 0
    z, zs = cache.quantize_token_int8(np.zeros((2, 128)))
    assert np.all(z == 0) and np.all(zs == 1)


def test_int8_codes_are_nearest():
    """Each code is the integer nearest x / scale (brute force over the 255
    codes), except within fp32 rounding of a half-way point."""
    x = _rng(2).standard_normal((40, 128)) * 0.7
    codes, scale = cache.quantize_token_int8(x)
    cand = np.arange(-127, 128, dtype=np.float64)
    for r in range(40):
        t = x[r] / float(scale[r])
        best = cand[np.abs(cand[None, :] - t[:, None]).argmin(axis=1)]
        off = codes[r] != best
        assert np.all(np.abs(np.abs(t[off] - np.floor(t[off])) - 0.5) < 1e-4)
    err = np.abs(cache.dequant_int8(codes, scale[:, None]) - x)
    assert np.all(err <= 0.5 * scale[:, None] * (1 + 1e-5))


def test_int8_append_round_trip():
    """Expected planes: K rotated (inverse rotation of the dequantised plane
    returns k within half a step), V transposed per token, scales per token."""
    from oracle.rope import rope3d, video_positions
    F, lh, lw, H, D = 2, 2, 3, 2, 128
    P = lh * lw
    k = _rng(3).standard_normal((F * P, H, D))
    v = _rng(4).standard_normal((F * P, H, D))
    kc, ks, vc, vs = cache.append_int8(k, v, 5, lh, lw, (16, 56, 56), 256.0)
    assert kc.shape == (F, H, P, D) and ks.shape == (F, H, P)
    assert vc.shape == (F, H, D, P) and vs.shape == (F, H, P)
    kr = rope3d(k, video_positions(5, F, lh, lw), (16, 56, 56), 256.0)
    kd = cache.dequant_int8(kc, ks[..., None]).transpose(0, 2, 1, 3).reshape(F * P, H, D)
    kstep = ks.transpose(0, 2, 1).reshape(F * P, H)[..., None]
    assert np.all(np.abs(kd - kr) <= 0.5 * kstep * 1.0001 + 1e-7)
    vd = cache.dequant_int8(vc, vs[:, :, None, :]).transpose(0, 3, 1, 2).reshape(F * P, H, D)
    assert np.all(np.abs(vd - v) <= 0.5 * vs.transpose(0, 2, 1).reshape(F * P, H)[..., None] * 1.0001)
    tk, tks, tv, tvs = cache.append_text_int8(k[:5], v[:5])
    assert tk.shape == (H, 5, D) and tks.shape == (H, 5) and tv.shape == (H, D, 5)
    np.testing.assert_array_equal(tk, cache.quantize_token_int8(k[:5].transpose(1, 0, 2))[0])
