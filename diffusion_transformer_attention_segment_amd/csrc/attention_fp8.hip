// segment_attention, e4m3 cache: fused Q-RoPE + Q quantisation + flash-style
// attention with fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, OCP e4m3 x e4m3,
// unit block scales) for both Q.K^T and P.V, fp32 accumulation.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// sections "How one segment is made" (the joint attention) and "The 4090
// preset" (the cache is quantised once per segment, one scale per group of
// values); "Hy-Nomas en una RTX 4090", section "El preset de una GPU" (the KV
// cache is stored narrow and computed at higher precision).
//
// Scales. The cache holds e4m3 codes with one fp32 scale per (frame, head)
// plane (per head for the text slot). A key tile never straddles a frame, so
// its K and V scales are uniform over the tile:
//   logit = (q_code . k_code) * q_scale[row] * k_scale[tile] * softmax scale
// -- one coefficient per lane and tile, folded into the exponent's FMA; and
//   O = sum_j p_j v_j = (vmax / 256) * sum_j P'_j v_code_j,
//   P'_j = p_j * 256 * v_scale[tile] / vmax,
// where vmax is the largest V scale among the session's kept planes for this
// head, so P' <= 256 * 2^slack stays inside e4m3 (max 448) and small
// probabilities keep 2^-8 more headroom above the e4m3 subnormal floor.
// Queries are rotated in fp32, then quantised per (row, head) in two parts:
// q_scale = amax / 448, y = q * 448 / amax, hi = e4m3(y), lo = e4m3(16 (y - hi)),
// q ~ (hi + lo / 16) q_scale. Q is never stored, so its split costs only a
// second MFMA per step (the low part enters through the MFMA's E8M0 block
// scale 2^-4) and removes most of the query's share of the fp8 error; the
// cache keeps one e4m3 code per value.
//
// Layout. One workgroup = 8 waves = 256 query rows of one head; each wave owns
// 32 rows. S^T = K Q^T with A = K rows (32 keys x 64 dims per MFMA), B = Q^T.
// Lane l of an S^T block b (32 keys) holds, in register r, the key
// 32*(l/32) + 16*b + r when A row r32 is loaded from key
// 32*((r32>>2)&1) + 16*b + 4*(r32>>3) + (r32&3): then the 32 probabilities a
// lane holds for a 64-key tile are the contiguous keys 32*(l/32) .. +31 -- the
// B-operand layout of O^T = V^T P^T -- and V^T (transposed in the cache) is
// read as 32 contiguous bytes per lane.
//
// Pipeline: one step per 64-key tile: PV of tile t-1 on the matrix pipe next to
// the softmax of tile t (max, exponentials against the running max, fp8
// packing), a wave-uniform branch for the rare running-max increase, then
// QK^T of tile t+1. K/V tiles go HBM -> registers -> a 4-stage LDS ring, one
// barrier per tile.
#include "attention_common.h"

namespace segattn {
namespace {

constexpr int BM = 256;
constexpr int BN = kKeyTile;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr int KS8 = kD + 16;           // LDS row stride of the K tile (bytes)
constexpr int VS8 = BN + 16;           // LDS row stride of the V^T tile (bytes)
constexpr int KT8 = BN * KS8;          // bytes of one K stage
constexpr int VT8 = kD * VS8;          // bytes of one V^T stage
constexpr float kSlack = 0.5f;         // log2 headroom of the lazy running max
constexpr float kPScale = 256.0f;      // probability pre-scale before e4m3

typedef int i32x8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8v& a, const i32x8v& b, const f32x16& c) {
  // A and B formats 0 = e4m3; E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Same, with the B operand scaled by 2^-4 through its E8M0 block scale (123):
// adds the low part of a split operand.
__device__ __forceinline__ f32x16 mfma_fp8_blo(const i32x8v& a, const i32x8v& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 123);
}

// two fp32 -> two e4m3 codes (round to nearest even) in the low or high half
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

// e4m3 code (low byte of c) -> fp32
__device__ __forceinline__ float fp8_decode(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  const float v = e == 0 ? static_cast<float>(m) * 0.001953125f
                         : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(v) | sign);
}

__device__ __forceinline__ i32x8v lds_read32(const uint8_t* p) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + 16);
  i32x8v r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

struct ChunkOffsets8 {
  uint32_t k;        // this thread's 16-byte chunk of a K tile
  uint32_t v_video;  // ... of a V^T tile, video plane stride
  uint32_t v_text;   // ... text plane stride
};

__device__ __forceinline__ void load_tile(const TileCursor& c, const ChunkOffsets8& off, bool video,
                                          u32x4& kr, u32x4& vr) {
  const __amdgpu_buffer_rsrc_t rk = tile_k_rsrc<1>(c);
  const __amdgpu_buffer_rsrc_t rv = tile_v_rsrc<1>(c);
  kr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off.k, 0, 0));
  vr = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, video ? off.v_video : off.v_text, 0, 0));
}

__device__ __forceinline__ void store_tile(uint8_t* Ks, uint8_t* Vs, int tid, const u32x4& kr,
                                           const u32x4& vr) {
  *reinterpret_cast<u32x4*>(Ks + (tid >> 3) * KS8 + (tid & 7) * 16) = kr;
  *reinterpret_cast<u32x4*>(Vs + (tid >> 2) * VS8 + (tid & 3) * 16) = vr;
}

// S^T of a 64-key tile: two 32-key blocks, two 64-dim steps each, each step
// with the high and the low (2^-4 scaled) part of the split query.
__device__ __forceinline__ void qk_tile(const uint8_t* Kst, const int* krow, int g,
                                        const i32x8v* qf, const i32x8v* ql, f32x16* s) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint8_t* kp = Kst + krow[b] * KS8 + 32 * g;
    const i32x8v k0 = lds_read32(kp), k1 = lds_read32(kp + 64);
    s[b] = mfma_fp8(k0, qf[0], f32x16{});
    s[b] = mfma_fp8_blo(k0, ql[0], s[b]);
    s[b] = mfma_fp8(k1, qf[1], s[b]);
    s[b] = mfma_fp8_blo(k1, ql[1], s[b]);
  }
}

// Tile max of S^T (32 keys per lane, both lane halves), raw dot-product units.
__device__ __forceinline__ float tile_max(const f32x16* s) {
  float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[0][r]), s[0][r + 1]);
  mx = fmaxf(mx, s[0][15]);
#pragma unroll
  for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, s[1][r]), s[1][r + 1]);
  return max_other_half(mx);
}

// Probabilities of a tile against the running max m (log2 units), summed into
// l, pre-scaled by pf and packed as e4m3 (32 bytes per lane, key order).
__device__ __forceinline__ void tile_probs(const f32x16* s, float coef, float m, float pf, float& l,
                                           i32x8v& p) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int b = w >> 2, r = (w & 3) * 4;
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[b][r], coef, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 1], coef, -m));
    const float p2 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 2], coef, -m));
    const float p3 = __builtin_amdgcn_exp2f(fmaf(s[b][r + 3], coef, -m));
    l += (p0 + p1) + (p2 + p3);
    uint32_t word = cvt_fp8x2<false>(p0 * pf, p1 * pf, 0u);
    word = cvt_fp8x2<true>(p2 * pf, p3 * pf, word);
    p[w] = static_cast<int>(word);
  }
}

__device__ __forceinline__ void mask_tile(f32x16* s, int nvalid, int g) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (32 * g + 16 * b + r >= nvalid) s[b][r] = -INFINITY;
}

// per-tile scalars carried through the load ring
struct TileInfo {
  int nvalid;
  float kscale;
  float vscale;
};

__device__ __forceinline__ TileInfo tile_info(const TileCursor& c) {
  TileInfo t;
  t.nvalid = cursor_nvalid(c);
  t.kscale = c.kscale;
  t.vscale = c.vscale;
  return t;
}

// First half of a step (one basic block): PV of tile t-1 (P'^T in p_prev,
// V^T stage vprev) on the matrix pipe next to the softmax of tile t (s_cur).
// Returns the tile max in log2 units.
__device__ __forceinline__ float pv_softmax(const uint8_t* vprev, int voff, const i32x8v& p_prev,
                                            f32x16* o, const f32x16* s_cur, float coef,
                                            float m_run, float pf, float& l_run, i32x8v& p_cur) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
    o[db] = mfma_fp8(lds_read32(vprev + voff + 32 * db * VS8), p_prev, o[db]);
  const float mt = tile_max(s_cur) * coef;
  tile_probs(s_cur, coef, m_run, pf, l_run, p_cur);
  asm volatile("" : "+v"(p_cur), "+v"(l_run));
  return mt;
}

__device__ __forceinline__ void rescale_step(float mt, float& m_run, float l_before, float& l_run,
                                             f32x16* o, const f32x16* s_cur, float coef, float pf,
                                             i32x8v& p_cur) {
  const bool need = mt > m_run + kSlack;
  const float mn = need ? mt : m_run;
  const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] *= alpha;
  m_run = mn;
  l_run = l_before * alpha;
  tile_probs(s_cur, coef, m_run, pf, l_run, p_cur);
}

__global__ __launch_bounds__(kThreads, 1) void attn_fp8_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kStages * KT8];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kStages * VT8];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  __shared__ float red[kWaves];

  const WorkTile wt = map_workgroup(a, BM);
  const AttnItemDev& I = a.items[wt.item];
  const int H = a.heads;
  const int h = wt.head;
  const int q0 = wt.q0;
  const int P = a.rope.P;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, r32 = lane & 31;

  ChunkOffsets8 off;
  off.k = static_cast<uint32_t>((tid >> 3) * kD + (tid & 7) * 16);
  off.v_video = static_cast<uint32_t>((tid >> 2) * P + (tid & 3) * 16);
  off.v_text = static_cast<uint32_t>((tid >> 2) * I.text_cap + (tid & 3) * 16);

  const int tpf = (P + BN - 1) / BN;
  const int ntiles = I.n_frames_kv * tpf + (I.n_text_kv + BN - 1) / BN;

  TileCursor lc;
  cursor_start<1>(lc, I, h, H, P);
  u32x4 kr, vr;
  TileInfo ti0 = tile_info(lc);
  load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);

  // largest V scale among the planes this (item, head) attends
  float vmax = 0.f;
  for (int i = tid; i < I.n_frames_kv; i += kThreads)
    vmax = fmaxf(vmax, I.v_scale[static_cast<size_t>(I.frames[i]) * H + h]);
  if (tid == 0 && I.n_text_kv > 0) vmax = fmaxf(vmax, I.v_text_scale[h]);
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o2));
  if (lane == 0) red[w] = vmax;
  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  for (int i = tid; i < VT8 / 16; i += kThreads)
    reinterpret_cast<u32x4*>(Vs + (kStages - 1) * VT8)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  vmax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) vmax = fmaxf(vmax, red[i]);

  // ---- Q: rotate in fp32, quantise per (row, head) to e4m3 ---------------------
  // lane holds dims 64*kk + 32*g + e (kk = 0, 1; e = 0..31) of its query row.
  // The query is split: qf = e4m3(q * 448 / amax), ql = e4m3(16 * residual), so
  // that qf + ql / 16 carries about 7 significant bits instead of 4.
  const int qrow = q0 + 32 * w + r32;
  i32x8v qf[2], ql[2];
  float q_scale;
  {
    bool video;
    int tpos, hpos, wpos;
    query_position(I, a.rope, qrow, &video, &tpos, &hpos, &wpos);
    float x[64];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        const int d0 = 64 * kk + 32 * g + 8 * ch;
        if (qrow < I.n_q)
          raw = *reinterpret_cast<const u32x4*>(I.q + (static_cast<size_t>(qrow) * H + h) * kD + d0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float xa = __uint_as_float(raw[m] << 16);
          float xb = __uint_as_float(raw[m] & 0xFFFF0000u);
          if (video) {
            const int pr = d0 / 2 + m;
            const int axis = ax[pr];
            const int pos = axis == 0 ? tpos : (axis == 1 ? hpos : wpos);
            float c, s;
            rope_cos_sin(pos, om[pr], &c, &s);
            const float ya = xa * c - xb * s;
            xb = xa * s + xb * c;
            xa = ya;
          }
          x[32 * kk + 8 * ch + 2 * m] = xa;
          x[32 * kk + 8 * ch + 2 * m + 1] = xb;
        }
      }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = max_other_half(amax);
    const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
    q_scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        float y[4], r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = x[32 * kk + 4 * wd + e] * inv;
        uint32_t hi = cvt_fp8x2<false>(y[0], y[1], 0u);
        hi = cvt_fp8x2<true>(y[2], y[3], hi);
        // residual against the decoded high part, scaled by 16 (|r| <= 448 / 16)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = 16.0f * (y[e] - fp8_decode(hi >> (8 * e)));
        uint32_t lo = cvt_fp8x2<false>(r[0], r[1], 0u);
        lo = cvt_fp8x2<true>(r[2], r[3], lo);
        qf[kk][wd] = static_cast<int>(hi);
        ql[kk][wd] = static_cast<int>(lo);
      }
  }

  // ---- prologue: tiles 0, 1 into LDS stages 0, 1; tile 2 in flight ----------
  store_tile(Ks, Vs, tid, kr, vr);
  TileInfo ti1 = ti0, ti2 = ti0;
  if (ntiles > 1) {
    cursor_next<1>(lc, I, h, H, P);
    ti1 = tile_info(lc);
    load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
    store_tile(Ks + KT8, Vs + VT8, tid, kr, vr);
  }
  if (ntiles > 2) {
    cursor_next<1>(lc, I, h, H, P);
    ti2 = tile_info(lc);
    load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
  }
  __syncthreads();

  int krow[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) krow[b] = 32 * ((r32 >> 2) & 1) + 16 * b + 4 * (r32 >> 3) + (r32 & 3);
  const int voff = r32 * VS8 + 32 * g;
  const float c2 = a.scale_log2 * q_scale;   // per-lane logit factor before the K scale
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float l_run = 0.f;

  f32x16 sc[2];
  qk_tile(Ks, krow, g, qf, ql, sc);
  if (ti0.nvalid < BN) mask_tile(sc, ti0.nvalid, g);
  float m_run = tile_max(sc) * (c2 * ti0.kscale);   // tile 0 always has a valid key
  i32x8v pa = {}, pb;
  const float pf_base = kPScale / vmax;

  // Tile t sits in stage t % 4. Step t: PV(t-1) beside softmax(t), then
  // QK^T(t+1) into the freed S registers (the other wave of the SIMD overlaps
  // its softmax with these MFMAs). Step t reads V of tile t-1 and K of tile
  // t+1, so tile t+2 goes to stage (t+2) % 4, last read before this tile's
  // barrier. Two steps per loop trip, so the P buffers swap roles without
  // copies.
  auto step = [&](int tt, i32x8v& p_prev, i32x8v& p_cur) __attribute__((always_inline)) {
    const uint8_t* Vprev = Vs + ((tt + kStages - 1) & (kStages - 1)) * VT8;
    const uint8_t* Knext = Ks + ((tt + 1) & (kStages - 1)) * KT8;
    const TileInfo cur = ti0;
    __syncthreads();
    TileInfo ti3 = ti0;
    if (tt + 2 < ntiles) {
      const int s2 = (tt + 2) & (kStages - 1);
      store_tile(Ks + s2 * KT8, Vs + s2 * VT8, tid, kr, vr);
      if (tt + 3 < ntiles) {
        cursor_next<1>(lc, I, h, H, P);
        ti3 = tile_info(lc);
        load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
      }
    }
    if (cur.nvalid < BN) mask_tile(sc, cur.nvalid, g);
    const float coef = c2 * cur.kscale;
    const float pf = pf_base * cur.vscale;
    const float l_before = l_run;
    const float mt = pv_softmax(Vprev, voff, p_prev, o, sc, coef, m_run, pf, l_run, p_cur);
    if (__any(mt > m_run + kSlack))
      rescale_step(mt, m_run, l_before, l_run, o, sc, coef, pf, p_cur);
    qk_tile(Knext, krow, g, qf, ql, sc);
    ti0 = ti1;
    ti1 = ti2;
    ti2 = ti3;
  };
#pragma unroll 1
  for (int t = 0; t < ntiles; t += 2) {
    step(t, pa, pb);
    if (t + 1 < ntiles) step(t + 1, pb, pa);
  }
  {
    const uint8_t* Vlast = Vs + ((ntiles - 1) & (kStages - 1)) * VT8;
    const i32x8v& p_last = (ntiles & 1) ? pb : pa;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      o[db] = mfma_fp8(lds_read32(Vlast + voff + 32 * db * VS8), p_last, o[db]);
  }

  // The output MFMAs compute across all lanes of the wave: keep them (and
  // everything feeding them) ahead of the per-row store branch below, where
  // lanes past the last query row are switched off.
  asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = vmax / (kPScale * l_tot);
  if (qrow < I.n_q) {
    uint16_t* orow = I.out + (static_cast<size_t>(qrow) * H + h) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * g;
        u32x2 v2;
        v2[0] = pack_bf16x2(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv);
        v2[1] = pack_bf16x2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = v2;
      }
    if (I.lse != nullptr && g == 0)
      I.lse[static_cast<size_t>(qrow) * H + h] = (m_run + __log2f(l_tot)) * 0.6931471805599453f;
  }
}

}  // namespace

int attention_block_m_fp8() { return BM; }

hipError_t launch_attention_fp8(AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_fp8_kernel, dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
