"""Cache planes: layout, byte counts and expected contents (oracle, test-only).

Sources: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
(ai.thesatyajit.com), sections "What 'world memory' stores" (K and V are each
2,048 wide per token and layer; BF16 costs 8,192 bytes per token per layer,
389 MB per 880-token latent frame over 54 layers) and "The 4090 preset" (the
INT8 cache spends a byte on each value and an FP32 scale on each token and
head: 4,224 bytes per token per layer; 18 kept frames are about 3.6 GB); section
"How one segment is made" (3D RoPE on keys; 880 tokens per latent frame).

Plane layout (the library's own design; the pages fix no layout). Per layer,
with H heads, D = head_dim, P = lat_h * lat_w tokens per latent frame and
PL = plane_slots(dtype, P) token slots per frame plane (P for bf16; P rounded
up to a multiple of 16 for the one-byte caches, so that every V^T row starts
16-byte aligned; slots p >= P hold zero V^T codes and zero int8 scales, and
their K rows are never read):

* K plane  [frame_capacity][H][PL][D]  element ((f*H + h)*PL + p)*D + c
* V plane  [frame_capacity][H][D][PL]  element ((f*H + h)*D + c)*PL + p
  (V is stored transposed per (frame, head): the P.V contraction runs over
  tokens, so tokens are the contiguous axis)
* text K   [H][text_capacity][D]      element (h*TC + i)*D + c
* text V   [H][D][text_capacity]      element (h*D + c)*TC + i
* fp8 (e4m3fn) planes use the same shapes with one byte per element, plus
  fp32 scales k_scale/v_scale [frame_capacity][H] and k_text_scale /
  v_text_scale [H].
* int8 planes (the pages' single-GPU format) use the same shapes with one
  signed byte per element, plus fp32 scales per token and head:
  k_scale/v_scale [frame_capacity][H][PL] and k_text_scale / v_text_scale
  [H][text_capacity].

Stored values. K is rotated by the 3D RoPE at its absolute position (frame f
for video token p of frame f; (0, 0, 0) for text) and rounded to the cache
format; V is stored unrotated. fp8 scale per (frame, head) plane (per head for
the text slot) = 2**e, e the smallest integer with amax <= 448 * 2**e over
that plane's (fp32) values, and at least -126 (amax == 0 gives scale 1);
codes = e4m3 round-nearest-even of x / 2**e, which no rounding precedes (the
division by a power of two is exact). A power of two is an fp32 scale like
any other; the choice lets fp8 matrix instructions apply the scale exactly
through their power-of-two block scales. The pages fix no fp8 format: the
e4m3 cache with fp32 scales per (frame, head) is the workload's own, and this
is the reading of how those scales are chosen.
int8 scale per (token, head) = amax / 127 over that token's head_dim values
in fp32 (amax == 0 gives scale 1); code = round-half-even of
x * (127 / amax) evaluated in fp32, clamped to [-127, 127] (symmetric: -128
is never used). The pages give the granularity and the byte count, not the
rounding; this is the plainest symmetric reading.
"""

import numpy as np

from . import numerics
from .rope import rope3d, video_positions, text_positions

E4M3_MAX = 448.0


# ---------------------------------------------------------------- byte counts
def bytes_per_token_per_layer(fmt, heads=16, head_dim=128):
    """K + V bytes of one token in one layer for a cache format.

    'bf16'            : 2 bytes per value
    'int8_token_head' : the pages' single-GPU format, 1 byte per value plus an
                        fp32 scale per token and head
    """
    width = heads * head_dim
    if fmt == "bf16":
        return 2 * width * 2
    if fmt == "int8_token_head":
        return 2 * (width + heads * 4)
    raise ValueError(fmt)


def plane_slots(dtype, P):
    """Token slots of one (frame, head) plane: P for bf16, else P rounded up
    to a multiple of 16."""
    if dtype == "bf16":
        return P
    if dtype in ("fp8", "int8"):
        return -(-P // 16) * 16
    raise ValueError(dtype)


def plane_bytes(dtype, heads, head_dim, P, frame_capacity, text_capacity):
    """Bytes of one layer's cache planes in this library's layout.

    dtype 'bf16', 'fp8' (fp32 scales per (frame, head) and per head for the
    text slot, for K and V) or 'int8' (fp32 scales per token and head).
    """
    PL = plane_slots(dtype, P)
    elems = 2 * heads * head_dim * (frame_capacity * PL + text_capacity)
    if dtype == "bf16":
        return 2 * elems
    if dtype == "fp8":
        return elems + 2 * 4 * heads * (frame_capacity + 1)
    return elems + 2 * 4 * heads * (frame_capacity * PL + text_capacity)


# --------------------------------------------------------------- layout maps
def k_offset(f, h, p, c, H, PL, D):
    """Element offset of K (frame f, head h, token p, dim c) in planes of PL
    token slots."""
    return ((f * H + h) * PL + p) * D + c


def v_offset(f, h, p, c, H, PL, D):
    """Element offset of V (frame f, head h, token p, dim c) in the
    transposed planes of PL token slots."""
    return ((f * H + h) * D + c) * PL + p


def text_k_offset(h, i, c, TC, D):
    return (h * TC + i) * D + c


def text_v_offset(h, i, c, TC, D):
    return (h * D + c) * TC + i


# ------------------------------------------------------ expected append (bf16)
def append_bf16(k_in, v_in, frame0, lat_h, lat_w, split, theta):
    """Expected bf16 plane contents for frames [frame0, frame0+F) of a segment.

    k_in, v_in: float64 [F*P, H, D] raw values (exact bf16 inputs), token
    order (t, h, w) raster. Returns (K [F, H, P, D], V [F, H, D, P]) as float64
    values that are exactly bf16: K = bf16(RoPE(k) in exact arithmetic), V a copy.
    """
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    P = lat_h * lat_w
    n, H, D = k_in.shape
    F = n // P
    pos = video_positions(frame0, F, lat_h, lat_w)
    kr = numerics.bf16_round(rope3d(k_in, pos, split, theta))
    K = kr.reshape(F, P, H, D).transpose(0, 2, 1, 3)
    V = v_in.reshape(F, P, H, D).transpose(0, 2, 3, 1)
    return K, V


def append_text_bf16(k_in, v_in):
    """Expected text slot (bf16): K [H, n, D] (identity rotation), V [H, D, n]."""
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    kr = numerics.bf16_round(rope3d(k_in, text_positions(k_in.shape[0])))
    return kr.transpose(1, 0, 2), v_in.transpose(1, 2, 0)


# ------------------------------------------------------- expected append (fp8)
E4M3_MIN_SCALE_EXP = -126


def plane_scale_exponent(amax):
    """The exponent e of a plane's scale 2**e: the smallest integer with
    amax <= 448 * 2**e, raised to -126 if smaller (0 for amax == 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = int(np.ceil(np.log2(amax / E4M3_MAX)))
    while amax > E4M3_MAX * 2.0 ** e:           # settle the exact boundary
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(e, E4M3_MIN_SCALE_EXP)


def quantize_plane_fp8(x):
    """Quantise one plane (any shape) of fp32-valued reals to e4m3 codes.

    Returns (codes uint8 same shape, scale float32). amax is the fp32 maximum
    magnitude, scale = 2**plane_scale_exponent(amax), code = e4m3 nearest-even
    of x / scale (an exact quotient), saturated.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0:
        return np.zeros(x32.shape, np.uint8), np.float32(1.0)
    e = plane_scale_exponent(amax)
    y = x32.astype(np.float64) * 2.0 ** -e
    return numerics.e4m3_encode(y), np.float32(2.0 ** e)


def append_fp8(k_in, v_in, frame0, lat_h, lat_w, split, theta):
    """Expected fp8 planes and scales for frames [frame0, frame0+F).

    K is rotated in exact arithmetic here and then quantised from its float32
    rounding; the kernel rotates in float32, so its K codes may differ from
    these by one code step near a rounding boundary. V is an exact input, so
    its codes and scales are fully determined.
    Returns (Kc [F,H,P,D] u8, Ks [F,H] f32, Vc [F,H,D,P] u8, Vs [F,H] f32).
    """
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    P = lat_h * lat_w
    n, H, D = k_in.shape
    F = n // P
    pos = video_positions(frame0, F, lat_h, lat_w)
    kr = rope3d(k_in, pos, split, theta).reshape(F, P, H, D).transpose(0, 2, 1, 3)
    vv = v_in.reshape(F, P, H, D).transpose(0, 2, 3, 1)
    Kc = np.zeros(kr.shape, np.uint8)
    Vc = np.zeros(vv.shape, np.uint8)
    Ks = np.zeros((F, H), np.float32)
    Vs = np.zeros((F, H), np.float32)
    for f in range(F):
        for h in range(H):
            Kc[f, h], Ks[f, h] = quantize_plane_fp8(kr[f, h])
            Vc[f, h], Vs[f, h] = quantize_plane_fp8(vv[f, h])
    return Kc, Ks, Vc, Vs


def append_text_fp8(k_in, v_in):
    """Expected fp8 text slot: (Kc [H,n,D], Ks [H], Vc [H,D,n], Vs [H])."""
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    n, H, D = k_in.shape
    kt = k_in.transpose(1, 0, 2)
    vt = v_in.transpose(1, 2, 0)
    Kc = np.zeros(kt.shape, np.uint8)
    Vc = np.zeros(vt.shape, np.uint8)
    Ks = np.zeros(H, np.float32)
    Vs = np.zeros(H, np.float32)
    for h in range(H):
        Kc[h], Ks[h] = quantize_plane_fp8(kt[h])
        Vc[h], Vs[h] = quantize_plane_fp8(vt[h])
    return Kc, Ks, Vc, Vs


def dequant(codes, scale):
    """Real value of fp8 codes times their plane scale (float64)."""
    return numerics.e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)


# ------------------------------------------------------ expected append (int8)
INT8_MAX = 127


def quantize_token_int8(x):
    """Quantise vectors (last axis: one token's head_dim values) to int8.

    Returns (codes int8 same shape, scale float32 [...]). In fp32: amax over
    the vector, scale = amax / 127, inv = 127 / amax (both 1 when amax is 0),
    code = rint(x * inv) clamped to [-127, 127]."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    nz = amax > 0
    safe = np.where(nz, amax, np.float32(1)).astype(np.float32)
    scale = np.where(nz, safe / np.float32(INT8_MAX), np.float32(1)).astype(np.float32)
    inv = np.where(nz, np.float32(INT8_MAX) / safe, np.float32(1)).astype(np.float32)
    y = (x32 * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.int8)
    return codes, scale


def append_int8(k_in, v_in, frame0, lat_h, lat_w, split, theta):
    """Expected int8 planes and per-token scales for frames [frame0, frame0+F).

    As for fp8, K is rotated in exact arithmetic and quantised from its
    float32 rounding (the kernel rotates in float32: a K code may differ by
    one step near a rounding boundary); V codes and scales are fully
    determined. Returns (Kc [F,H,P,D] i8, Ks [F,H,P] f32, Vc [F,H,D,P] i8,
    Vs [F,H,P] f32)."""
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    P = lat_h * lat_w
    n, H, D = k_in.shape
    F = n // P
    pos = video_positions(frame0, F, lat_h, lat_w)
    kr = rope3d(k_in, pos, split, theta).reshape(F, P, H, D).transpose(0, 2, 1, 3)
    kc, ks = quantize_token_int8(kr)
    vt = v_in.reshape(F, P, H, D).transpose(0, 2, 1, 3)            # [F, H, P, D]
    vc, vs = quantize_token_int8(vt)
    return kc, ks, np.ascontiguousarray(vc.transpose(0, 1, 3, 2)), vs


def append_text_int8(k_in, v_in):
    """Expected int8 text slot: (Kc [H,n,D], Ks [H,n], Vc [H,D,n], Vs [H,n])."""
    k_in = np.asarray(k_in, dtype=np.float64)
    v_in = np.asarray(v_in, dtype=np.float64)
    kc, ks = quantize_token_int8(k_in.transpose(1, 0, 2))
    vc, vs = quantize_token_int8(v_in.transpose(1, 0, 2))
    return kc, ks, np.ascontiguousarray(vc.transpose(0, 2, 1)), vs


def dequant_int8(codes, scale):
    """Real value of int8 codes times their per-token scale (float64); scale
    broadcasts over the codes' token axis as the caller arranges."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)
