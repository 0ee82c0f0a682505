// kv_append / text_append kernels: 3D RoPE on K, cache-plane stores of K and
// (transposed) V, bf16, e4m3 + per-(frame, head) scales, or int8 + per-(token,
// head) scales.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// sections "How one segment is made" (RoPE split [16, 56, 56] over t, h, w)
// and "Writing the segment into memory" (the finished segment's K/V are
// stored); "The 4090 preset" (the cache is quantised once per segment).
//
// HBM-bound: per token and head the kernels read 2 x 256 B of bf16 input and
// write 2 x 256 B (bf16) or 2 x 128 B (e4m3, int8; int8 adds 2 x 4 B of
// scales) of cache. Blocks run heads
// fastest, so that concurrent blocks read the same tokens' rows of all heads
// (4 KB contiguous per token). The bf16 kernel transposes V through LDS and
// stores 16-byte runs of V^T rows; it tabulates the cos/sin of its tile (the
// frame's t band, the rows it spans, every column) in LDS first. The e4m3
// kernel holds one (frame, head) plane per block (the scale needs the plane's
// amax); it tabulates the rotation angles in LDS once per block (they depend
// on the band position and the pair only) and transposes V through an LDS
// tile as well, 128 tokens at a time.
#include "device_common.h"

namespace segattn {
namespace {

constexpr int kTileTok = 64;          // tokens per bf16 block tile
constexpr int kVtStride = kD + 8;     // LDS row stride (elements) of the V tile
constexpr int kLutMax = 4096;         // rotation table entries (cos, sin) within the LDS budget
constexpr int kTileLutMax = 2048;     // entries of a bf16 tile's table

// latent rows a 64-token tile can span (tiles start at any token of a row)
__host__ __device__ constexpr int tile_rows(int lat_w) { return (kTileTok - 1) / lat_w + 2; }

// Rotate the 8 bf16 values of one 16-byte chunk (dims ch*8 .. ch*8+7) of a key
// at (t, h, w), in fp32, and return them rounded to bf16.
__device__ __forceinline__ void rotate_chunk(const u32x4& x, int ch, int t, int hh, int ww,
                                             const double* om, const int* ax, float* y) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t wv = x[m];
    float a = __uint_as_float(wv << 16);
    float b = __uint_as_float(wv & 0xFFFF0000u);
    int pr = ch * 4 + m;
    int axis = ax[pr];
    int pos = axis == 0 ? t : (axis == 1 ? hh : ww);
    float c, s;
    rope_cos_sin(pos, om[pr], &c, &s);
    y[2 * m] = a * c - b * s;
    y[2 * m + 1] = a * s + b * c;
  }
}

// ---- RoPE table ------------------------------------------------------------------
struct LutShape {
  int nt, nh, nw;   // pairs per band (t, h, w)
  int lat_h;
  int size;         // entries: nt + lat_h * nh + lat_w * nw
};

__device__ __forceinline__ LutShape lut_shape(const RopeParams& r) {
  LutShape s;
  s.nt = r.split0 / 2;
  s.nh = r.split1 / 2;
  s.nw = r.split2 / 2;
  s.lat_h = r.P / r.lat_w;
  s.size = s.nt + s.lat_h * s.nh + r.lat_w * s.nw;
  return s;
}

// Entry i: t-band pair i at position t, then [hh][j] for the h band, then
// [ww][j] for the w band; each from the same fp64-reduced angle as the direct
// evaluation (rope_cos_sin), so a table lookup and the direct path agree
// bit for bit.
__device__ void build_lut(float2* lut, const LutShape& s, int t, const RopeParams& r, int tid,
                          int nthreads, int row0 = 0) {
  for (int i = tid; i < s.size; i += nthreads) {
    int pair, pos;
    if (i < s.nt) {
      pair = i;
      pos = t;
    } else if (i < s.nt + s.lat_h * s.nh) {
      const int j = i - s.nt;
      const int rr = j / s.nh;
      pos = row0 + rr;
      pair = s.nt + (j - rr * s.nh);
    } else {
      const int j = i - s.nt - s.lat_h * s.nh;
      pos = j / s.nw;
      pair = s.nt + s.nh + (j - pos * s.nw);
    }
    int axis;
    const double om = rope_omega(pair, r, &axis);
    float c, sn;
    rope_cos_sin(pos, om, &c, &sn);
    lut[i] = make_float2(c, sn);
  }
}

__device__ __forceinline__ float2 lut_get(const float2* lut, const LutShape& s, int pair, int hh,
                                          int ww) {
  if (pair < s.nt) return lut[pair];
  if (pair < s.nt + s.nh) return lut[s.nt + hh * s.nh + (pair - s.nt)];
  return lut[s.nt + s.lat_h * s.nh + ww * s.nw + (pair - s.nt - s.nh)];
}

// The 8 values of one 16-byte chunk (dims 8 ch .. 8 ch + 7) of a key at
// (t, hh, ww): rotated in fp32 (cos/sin from the table when given, else
// evaluated), or, for text keys, unrotated.
template <bool kLut>
__device__ __forceinline__ void key_chunk(const u32x4& x, int ch, int t, int hh, int ww,
                                          bool rotate, const float2* lut, const LutShape& ls,
                                          const RopeParams& r, float* y) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float a = __uint_as_float(x[m] << 16);
    const float b = __uint_as_float(x[m] & 0xFFFF0000u);
    if (!rotate) {
      y[2 * m] = a;
      y[2 * m + 1] = b;
      continue;
    }
    const int pr = ch * 4 + m;
    float c, s;
    if constexpr (kLut) {
      const float2 cs = lut_get(lut, ls, pr, hh, ww);
      c = cs.x;
      s = cs.y;
    } else {
      int axis;
      const double om = rope_omega(pr, r, &axis);
      rope_cos_sin(axis == 0 ? t : (axis == 1 ? hh : ww), om, &c, &s);
    }
    y[2 * m] = a * c - b * s;
    y[2 * m + 1] = a * s + b * c;
  }
}

__device__ __forceinline__ u32x4 load_chunk(const uint16_t* base, size_t off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// ---- e4m3 ------------------------------------------------------------------------
// Exponent e of a plane's scale 2^e: the least integer with amax <= 448 * 2^e,
// at least -126 (0 when amax is 0). With 448 = 1.75 * 2^8 and amax = m * 2^k,
// 1 <= m < 2: e = k - 8, or k - 7 when m > 1.75 (mantissa field above 0x600000).
__device__ __forceinline__ int e4m3_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int biased = static_cast<int>(b >> 23);
  if (biased == 0) return -126;                 // below 2^-126: the floor
  const int e = biased - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -126 ? -126 : e;
}

// 2^e as an fp32 value (e in [-126, 127])
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float(static_cast<uint32_t>(e + 127) << 23); }

// Four fp32 values already scaled into +-448 (by 2^-e) -> four OCP
// e4m3fn codes, first value in the low byte, by the hardware conversion:
// round to nearest even, values below 2^-6 to the nearest multiple of 2^-9.
// In this range nothing overflows.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}

__device__ __forceinline__ float block_max(float v, float* red, int nthreads) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < nthreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// kLut: the block tabulates the cos/sin its 64 tokens need (the frame's t
// band, the h band of the latent rows the tile spans, the w band of every
// column) in LDS, about 1,200 entries at a 22 x 40 grid against 4,096 direct
// evaluations; else each pair is evaluated directly.
template <bool kLut>
__global__ __launch_bounds__(256) void append_bf16_kernel(const AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileTok * kVtStride];
  __shared__ double om[kLut ? 1 : kD / 2];
  __shared__ int ax[kLut ? 1 : kD / 2];
  __shared__ float2 lut[kLut ? kTileLutMax : 1];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.y * kTileTok;
  const int fr = blockIdx.z;
  const int h = blockIdx.x;
  const int H = a.heads;
  const int f = a.frame0 + fr;
  const int lat_w = a.rope.lat_w;
  const int row0 = p0 / lat_w;
  LutShape ls = lut_shape(a.rope);
  if constexpr (kLut) {
    ls.lat_h = tile_rows(lat_w);
    ls.size = ls.nt + ls.lat_h * ls.nh + lat_w * ls.nw;
    if (!a.is_text) build_lut(lut, ls, f, a.rope, tid, 256, row0);
  } else if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();
  const size_t plane = static_cast<size_t>(a.plane_len) * kD;
  uint16_t* kdst = static_cast<uint16_t*>(a.k) + (static_cast<size_t>(f) * H + h) * plane;
  uint16_t* vdst = static_cast<uint16_t*>(a.v) + (static_cast<size_t>(f) * H + h) * plane;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int tok = c >> 4, ch = c & 15;
    const int p = p0 + tok;
    u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (p < a.n_tok) {
      const size_t in_off = (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
      kx = *reinterpret_cast<const u32x4*>(a.k_in + in_off);
      vx = *reinterpret_cast<const u32x4*>(a.v_in + in_off);
      u32x4 ky = kx;
      if (!a.is_text) {
        float y[8];
        if constexpr (kLut)
          key_chunk<true>(kx, ch, f, p / lat_w - row0, p % lat_w, true, lut, ls, a.rope, y);
        else
          rotate_chunk(kx, ch, f, p / lat_w, p % lat_w, om, ax, y);
#pragma unroll
        for (int m = 0; m < 4; ++m) ky[m] = pack_bf16x2(y[2 * m], y[2 * m + 1]);
      }
      *reinterpret_cast<u32x4*>(kdst + static_cast<size_t>(p) * kD + ch * 8) = ky;
    }
    *reinterpret_cast<u32x4*>(&vt[tok * kVtStride + ch * 8]) = vx;
  }
  __syncthreads();
  // transposed V: row d, tokens p0 + 8*tc .. +7
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int d = c >> 3, tc = c & 7;
    const int p = p0 + 8 * tc;
    if (p < a.plane_len) {
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t lo = vt[(8 * tc + 2 * m) * kVtStride + d];
        uint32_t hi = vt[(8 * tc + 2 * m + 1) * kVtStride + d];
        o[m] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(vdst + static_cast<size_t>(d) * a.plane_len + p) = o;
    }
  }
}

constexpr int kFp8Threads = 512;
constexpr int kVtTok = 128;              // tokens per V^T tile
// LDS row stride of the V^T tile (words): odd, so that the word stores of the
// 16 chunks of a token quad (rows 8 apart) fall in 8 banks; rows are read out
// as 4-byte words
constexpr int kVtWords = kVtTok / 4 + 1;

// One block per (frame, head) plane (or per head of the text slot): pass 1
// finds amax of the rotated K and of V, pass 2 quantises and stores (K rows of
// 8-byte chunks; V^T rows in 4-byte words of 4 consecutive tokens). The
// scale of a plane is the least power of two 2^e with amax <= 448 * 2^e.
template <bool kLut>
__global__ __launch_bounds__(kFp8Threads) void append_fp8_kernel(const AppendArgs a) {
  __shared__ float2 lut_mem[kLutMax];
  __shared__ float red[kFp8Threads / 64];
  __shared__ __align__(16) uint32_t vt_tile[kD * kVtWords];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int fr = blockIdx.y;
  const int H = a.heads;
  const int f = a.frame0 + fr;
  const bool rotate = !a.is_text;
  const LutShape ls = lut_shape(a.rope);
  if constexpr (kLut) {
    build_lut(lut_mem, ls, f, a.rope, tid, kFp8Threads);
    __syncthreads();
  }
  const float2* lut = lut_mem;
  const int lat_w = a.rope.lat_w;
  const int n_chunks = a.n_tok * 16;
  auto in_off = [&](int p, int ch) {
    return (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
  };
  float amk = 0.f, amv = 0.f;
#pragma unroll 2
  for (int c = tid; c < n_chunks; c += kFp8Threads) {
    const int p = c >> 4, ch = c & 15;
    const u32x4 kx = load_chunk(a.k_in, in_off(p, ch));
    const u32x4 vx = load_chunk(a.v_in, in_off(p, ch));
    float y[8];
    key_chunk<kLut>(kx, ch, f, p / lat_w, p % lat_w, rotate, lut, ls, a.rope, y);
#pragma unroll
    for (int m = 0; m < 8; ++m) amk = fmaxf(amk, fabsf(y[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      amv = fmaxf(amv, fabsf(__uint_as_float(vx[m] << 16)));
      amv = fmaxf(amv, fabsf(__uint_as_float(vx[m] & 0xFFFF0000u)));
    }
  }
  amk = block_max(amk, red, kFp8Threads);
  amv = block_max(amv, red, kFp8Threads);
  // power-of-two scales: the codes are the e4m3 roundings of x * 2^-e, an
  // exact product
  const int ek = e4m3_scale_exp(amk), ev = e4m3_scale_exp(amv);
  const float ik = pow2f(-ek), iv = pow2f(-ev);
  if (tid == 0) {
    a.k_scale[static_cast<size_t>(f) * H + h] = pow2f(ek);
    a.v_scale[static_cast<size_t>(f) * H + h] = pow2f(ev);
  }
  const size_t plane = static_cast<size_t>(a.plane_len) * kD;
  uint8_t* kdst = static_cast<uint8_t*>(a.k) + (static_cast<size_t>(f) * H + h) * plane;
  uint8_t* vdst = static_cast<uint8_t*>(a.v) + (static_cast<size_t>(f) * H + h) * plane;
#pragma unroll 2
  for (int c = tid; c < n_chunks; c += kFp8Threads) {
    const int p = c >> 4, ch = c & 15;
    float y[8];
    key_chunk<kLut>(load_chunk(a.k_in, in_off(p, ch)), ch, f, p / lat_w, p % lat_w, rotate, lut,
                    ls, a.rope, y);
    u32x2 o;
#pragma unroll
    for (int m = 0; m < 2; ++m)
      o[m] = e4m3x4(y[4 * m] * ik, y[4 * m + 1] * ik, y[4 * m + 2] * ik, y[4 * m + 3] * ik);
    *reinterpret_cast<u32x2*>(kdst + static_cast<size_t>(p) * kD + ch * 8) = o;
  }
  // V^T through LDS, 128 tokens at a time. Load: thread = (token quad jq,
  // chunk ch), ch fastest, so that 16 lanes read one token's 256 bytes; its 4
  // tokens x 8 dims become 8 words (4 tokens of one dim each) in the LDS tile
  // [dim][token]. Store: each V^T row's 128 bytes leave as 8 runs of 16 bytes.
  // plane_len % 16 == 0; tokens past n_tok store the code of +0.
  static_assert(kFp8Threads == 512, "one (quad, chunk) item per thread per 128-token tile");
  for (int t0 = 0; t0 < a.plane_len; t0 += kVtTok) {
    {
      const int ch = tid & 15, jq = tid >> 4;
      const int p = t0 + 4 * jq;
      u32x4 vx[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        vx[q] = p + q < a.n_tok ? load_chunk(a.v_in, in_off(p + q, ch)) : u32x4{0u, 0u, 0u, 0u};
      __syncthreads();               // the previous tile's rows have been read out
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        auto lo = [&](int q) { return __uint_as_float(vx[q][m] << 16) * iv; };
        auto hi = [&](int q) { return __uint_as_float(vx[q][m] & 0xFFFF0000u) * iv; };
        vt_tile[(8 * ch + 2 * m) * kVtWords + jq] = e4m3x4(lo(0), lo(1), lo(2), lo(3));
        vt_tile[(8 * ch + 2 * m + 1) * kVtWords + jq] = e4m3x4(hi(0), hi(1), hi(2), hi(3));
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int idx = tid + r * kFp8Threads;
      const int d = idx >> 3, pc = idx & 7;
      if (t0 + 16 * pc < a.plane_len) {
        const uint32_t* w = &vt_tile[d * kVtWords + 4 * pc];
        *reinterpret_cast<u32x4*>(vdst + static_cast<size_t>(d) * a.plane_len + t0 + 16 * pc) =
            u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
}

}  // namespace

// the rotation table serves video planes whose table fits the LDS budget
static bool use_lut(const AppendArgs& a) {
  const RopeParams& r = a.rope;
  const int64_t size = r.split0 / 2 + static_cast<int64_t>(r.P / r.lat_w) * (r.split1 / 2) +
                       static_cast<int64_t>(r.lat_w) * (r.split2 / 2);
  return !a.is_text && size <= kLutMax;
}

namespace {

// ---- int8 with a scale per token and head ---------------------------------------
// One block = 64 tokens of one (frame, head) plane, 256 threads. A row of 16
// lanes owns four consecutive tokens, each lane 8 dims of each. Per (token,
// head) row, in fp32: rotate K (video), amax over the 128 dims, scale =
// amax / 127, inv = 127 / amax (both 1 when amax is 0), code = rint(x * inv)
// (|x * inv| <= 127 (1 + 2^-24), so no code passes +-127 and no clamp is
// needed). The amax of a row is a max across its 16 lanes by DPP; the two
// divisions of the four rows a lane row quantises at a time are spread over
// its lanes (lanes 0-3: inv of rows 0-3, lanes 4-7: their scales) and the
// inverses broadcast back. K codes go out as 8-byte runs of the row, V codes
// through an LDS [dim][token] tile, four tokens to a word, so that V^T rows
// leave as 16-byte runs. Tokens from n_tok to the plane's end (the padded
// slots) get zero codes and zero scales.
constexpr int kI8Tok = 64;
// LDS row stride (bytes) of the V^T tile (a word of four tokens per store)
constexpr int kI8Stride = kI8Tok + 4;
// 1.5 * 2^23: fl(t + kRoundMagic) for |t| < 2^22 is kRoundMagic + rint(t)
// (rounding to nearest even), and its low byte is rint(t) as a two's
// complement byte
constexpr float kRoundMagic = 12582912.0f;

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}

// max over the 16 lanes of a row of non-negative fp32 values, as bit patterns
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1, 0, 3, 2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2, 3, 0, 1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));   // row_mirror
  return v;
}

// lane n of each row of 16 to the whole row
template <int kN>
__device__ __forceinline__ float row16_bcast(float v) {
  return __uint_as_float(dpp_u32<0x150 + kN>(__float_as_uint(v)));
}

__device__ __forceinline__ uint32_t amax8(const float* x) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
  return __float_as_uint(am);
}

// kRoundMagic + rint(x * inv): the product rounded to fp32 first, then to an
// integer (two roundings, as the definition; no fused multiply-add)
__device__ __forceinline__ uint32_t code_bits(float x, float inv) {
#pragma clang fp contract(off)
  const float t = x * inv;
  return __float_as_uint(t + kRoundMagic);
}

// the low bytes of four words, first in the low byte
__device__ __forceinline__ uint32_t low_bytes4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Four rows (one per token of a lane row, values x[i][0..7] in this lane):
// inv[i] for each row, in every lane; scale of row (lane & 3) in lanes 4-7 of
// the lane row (returned, meaningful there).
__device__ __forceinline__ float row_scales4(const float (*x)[8], int lane, float* inv) {
  uint32_t am[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) am[i] = row16_max(amax8(x[i]));
  const int r = lane & 3;
  const float a = __uint_as_float(r == 0 ? am[0] : r == 1 ? am[1] : r == 2 ? am[2] : am[3]);
  const bool scale_lane = (lane & 4) != 0;   // else an inverse lane
  const float num = scale_lane ? a : 127.0f, den = scale_lane ? 127.0f : a;
  const float q = a > 0.f ? num / den : 1.0f;   // one correctly rounded division
  inv[0] = row16_bcast<0>(q);
  inv[1] = row16_bcast<1>(q);
  inv[2] = row16_bcast<2>(q);
  inv[3] = row16_bcast<3>(q);
  return q;
}

// kLut: the tile's cos/sin table in LDS, as for the bf16 kernel
template <bool kLut>
__global__ __launch_bounds__(256) void append_int8_kernel(const AppendArgs a) {
  static_assert(kI8Tok == kTileTok, "the tile table covers 64 tokens");
  __shared__ __attribute__((aligned(16))) uint8_t vt[kD * kI8Stride];
  __shared__ double om[kLut ? 1 : kD / 2];
  __shared__ int ax[kLut ? 1 : kD / 2];
  __shared__ float2 lut[kLut ? kTileLutMax : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 15, grp = tid >> 4;
  const int p0 = blockIdx.y * kI8Tok;
  const int fr = blockIdx.z;
  const int h = blockIdx.x;
  const int H = a.heads;
  const int f = a.frame0 + fr;
  const int lat_w = a.rope.lat_w;
  const int row0 = p0 / lat_w;
  LutShape ls = lut_shape(a.rope);
  if constexpr (kLut) {
    ls.lat_h = tile_rows(lat_w);
    ls.size = ls.nt + ls.lat_h * ls.nh + lat_w * ls.nw;
    build_lut(lut, ls, f, a.rope, tid, 256, row0);
  } else if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  const size_t pl = static_cast<size_t>(f) * H + h;
  int8_t* kdst = static_cast<int8_t*>(a.k) + pl * a.plane_len * kD;
  int8_t* vdst = static_cast<int8_t*>(a.v) + pl * a.plane_len * kD;
  // the lane row's tokens t0 .. t0 + 3: all inside the plane or all past it
  // (plane lengths of one-byte caches are multiples of 16)
  const int t0 = p0 + 4 * grp;
  const bool in_plane = t0 < a.plane_len;
  u32x4 kx[4], vx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kx[i] = vx[i] = u32x4{0u, 0u, 0u, 0u};
    if (t0 + i < a.n_tok) {
      const size_t in_off = (static_cast<size_t>(fr * a.n_tok + t0 + i) * H + h) * kD + lane * 8;
      kx[i] = *reinterpret_cast<const u32x4*>(a.k_in + in_off);
      vx[i] = *reinterpret_cast<const u32x4*>(a.v_in + in_off);
    }
  }
  __syncthreads();   // the rotation table
  // ---- K: rotate, scales, codes (8-byte runs of each token's row)
  {
    float y[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = t0 + i;
      if constexpr (kLut) {
        key_chunk<true>(kx[i], lane, f, p / lat_w - row0, p % lat_w, true, lut, ls, a.rope, y[i]);
      } else if (!a.is_text) {
        rotate_chunk(kx[i], lane, f, p / lat_w, p % lat_w, om, ax, y[i]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          y[i][2 * m] = __uint_as_float(kx[i][m] << 16);
          y[i][2 * m + 1] = __uint_as_float(kx[i][m] & 0xFFFF0000u);
        }
      }
    }
    float inv[4];
    const float q = row_scales4(y, lane, inv);
    if (in_plane) {
      if ((lane & 12) == 4) {   // lanes 4-7: the scales of tokens t0 .. t0 + 3
        const int p = t0 + (lane & 3);
        a.k_scale[pl * a.plane_len + p] = p < a.n_tok ? q : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t c[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) c[m] = code_bits(y[i][m], inv[i]);
        *reinterpret_cast<uint2*>(kdst + static_cast<size_t>(t0 + i) * kD + lane * 8) =
            make_uint2(low_bytes4(c[0], c[1], c[2], c[3]), low_bytes4(c[4], c[5], c[6], c[7]));
      }
    }
  }
  // ---- V: scales, codes as words of four tokens of one dim in the V^T tile
  {
    float z[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        z[i][2 * m] = __uint_as_float(vx[i][m] << 16);
        z[i][2 * m + 1] = __uint_as_float(vx[i][m] & 0xFFFF0000u);
      }
    float inv[4];
    const float q = row_scales4(z, lane, inv);
    if (in_plane && (lane & 12) == 4) {
      const int p = t0 + (lane & 3);
      a.v_scale[pl * a.plane_len + p] = p < a.n_tok ? q : 0.f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *reinterpret_cast<uint32_t*>(&vt[(lane * 8 + m) * kI8Stride + 4 * grp]) =
          low_bytes4(code_bits(z[0][m], inv[0]), code_bits(z[1][m], inv[1]),
                     code_bits(z[2][m], inv[2]), code_bits(z[3][m], inv[3]));
  }
  __syncthreads();
  // V^T rows: dim d, tokens p0 + 16 q .. + 15 (16-byte runs)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    const int d = c >> 2, q = c & 3;
    const int p = p0 + 16 * q;
    if (p < a.plane_len) {
      const uint32_t* row = reinterpret_cast<const uint32_t*>(&vt[d * kI8Stride + 16 * q]);
      *reinterpret_cast<u32x4*>(vdst + static_cast<size_t>(d) * a.plane_len + p) =
          u32x4{row[0], row[1], row[2], row[3]};
    }
  }
}

}  // namespace

// video planes whose 64-token tile table fits kTileLutMax entries
static bool use_tile_lut(const AppendArgs& a) {
  const RopeParams& r = a.rope;
  const int64_t size = r.split0 / 2 + static_cast<int64_t>(tile_rows(r.lat_w)) * (r.split1 / 2) +
                       static_cast<int64_t>(r.lat_w) * (r.split2 / 2);
  return !a.is_text && size <= kTileLutMax;
}

hipError_t launch_append_int8(const AppendArgs& a, hipStream_t s) {
  dim3 grid(a.heads, (a.plane_len + kI8Tok - 1) / kI8Tok, a.n_frames);   // heads fastest
  if (use_tile_lut(a))
    hipLaunchKernelGGL(append_int8_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_int8_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s) {
  // heads fastest: concurrent blocks read the same tokens' rows of all heads
  dim3 grid(a.heads, (a.plane_len + kTileTok - 1) / kTileTok, a.n_frames);
  if (use_tile_lut(a))
    hipLaunchKernelGGL(append_bf16_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_bf16_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s) {
  dim3 grid(a.heads, a.n_frames);   // heads fastest, as for bf16
  if (use_lut(a))
    hipLaunchKernelGGL(append_fp8_kernel<true>, grid, dim3(kFp8Threads), 0, s, a);
  else
    hipLaunchKernelGGL(append_fp8_kernel<false>, grid, dim3(kFp8Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
