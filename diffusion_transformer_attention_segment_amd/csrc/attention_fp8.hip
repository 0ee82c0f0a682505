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
//   logit (log2 units) = (q_code . k_code) * coef,
//   coef = q_scale[row] * k_scale[tile] * softmax scale * log2(e);
//   P'_j = exp2(x_j), x_j = logit_j + log2(pf) - m, pf = 256 * v_scale[tile] / vmax,
// i.e. P'_j = p_j * pf with p_j = exp2(logit_j - m) -- the probability scale
// rides in the exponent's FMA offset, one FMA per key. Then
//   O = sum_j p_j v_j = (vmax / 256) * sum_j P'_j v_code_j,
// where vmax is the largest V scale among the session's kept planes for this
// head. The running max m moves (rarely) when some x passes 8.5, i.e. P'
// would pass 362 (e4m3 max 448), to put the largest x at 8.
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
// Pipeline: one step per 64-key tile. Its 12 MFMAs (PV of tile t-1: 4; QK^T
// of tile t+1: 2 blocks x 2 k-steps x high/low query parts) are issued slot
// by slot next to the softmax of tile t, eight 4-key words of exp2 + e4m3
// packing. S^T is computed in place: block 0 of tile t+1 replaces block 0 of
// tile t once its words are packed, block 1 after the rescale check. Tiles go
// HBM -> LDS directly (buffer loads with the LDS flag) two tiles ahead into a
// 4-stage ring, one barrier per tile.
#include "attention_common.h"

namespace segattn {
namespace {

constexpr int BM = 256;
static_assert(BM == SA_SPARSE_QUERY_BLOCK, "a work tile reads one block list");
constexpr int BN = kKeyTile;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr int KS8 = kD + 16;           // LDS row stride of the K tile (bytes)
constexpr int VS8 = BN + 16;           // LDS row stride of the V^T tile (bytes)
constexpr int KT8 = BN * KS8;          // bytes of one K stage
constexpr int VT8 = kD * VS8;          // bytes of one V^T stage
constexpr float kPScale = 256.0f;      // probability pre-scale before e4m3 (log2: 8)
constexpr float kPTarget = 8.0f;       // log2 of P' for the largest key after a rescale
constexpr float kTrigger = 8.5f;       // log2 of P' above which the running max moves

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

// K tile: 64 rows of 9 slots (128 data bytes + pad); V^T tile: 128 rows of 5
// slots (64 data bytes + pad).
__device__ __forceinline__ int dma_k8(const TileCursor& c, uint8_t* stage, int w) {
  return dma_tile<BN, KS8 / 16>(tile_k_rsrc<1>(c), stage, kD, w);
}
__device__ __forceinline__ int dma_v8(const TileCursor& c, uint8_t* stage, int w) {
  return dma_tile<kD, VS8 / 16>(tile_v_rsrc<1>(c), stage, static_cast<uint32_t>(c.vstride), w);
}


// Keys at or past nvalid get -inf. (Compared as 16 b + r >= nvalid - 32 g: one
// per-lane value against immediates, rather than 32 per-lane key indices the
// compiler would keep in registers across the loop.)
__device__ __forceinline__ void mask_tile(f32x16* s, int nvalid, int g) {
  const int lim = nvalid - 32 * g;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (16 * b + r >= lim) s[b][r] = -INFINITY;
}

// Timed text windows on a tile: `word` is this lane's visibility word (bit b:
// key 32 g + b of the tile), register r of block b holds key 32 g + 16 b + r.
__device__ __forceinline__ void window_mask_tile(f32x16* s, uint32_t word) {
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[b][r] = keep_if_bit(s[b][r], word, 16 * b + r);
}

// per-tile scalars carried through the load ring
struct TileInfo {
  int nvalid;   // valid-key count, sign bit set on a text tile under windows
  float kscale;
  float vscale;
};

__device__ __forceinline__ TileInfo tile_info(const TileCursor& c, int flag_fi) {
  TileInfo t;
  t.nvalid = cursor_mask_code(c, flag_fi);
  t.kscale = c.kscale;
  t.vscale = c.vscale;
  return t;
}

// Word w (0..3) of one 32-key block: keys 4w .. 4w+3 of the block (registers
// 4w ..), as P' = exp2(x) with x = s * coef + off, packed e4m3. Accumulates the
// fp32 sum and the max of x.
__device__ __forceinline__ uint32_t prob_word_blk(const f32x16& s, int w, float coef, float off,
                                                  float& l, float& mx) {
  const int r = w * 4;
  const float x0 = fmaf(s[r], coef, off), x1 = fmaf(s[r + 1], coef, off);
  const float x2 = fmaf(s[r + 2], coef, off), x3 = fmaf(s[r + 3], coef, off);
  mx = fmaxf(fmaxf(mx, x0), fmaxf(x1, fmaxf(x2, x3)));
  const float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
  const float p2 = __builtin_amdgcn_exp2f(x2), p3 = __builtin_amdgcn_exp2f(x3);
  uint32_t word = cvt_fp8x2<false>(p0, p1, 0u);
  word = cvt_fp8x2<true>(p2, p3, word);
  l += (p0 + p1) + (p2 + p3);
  return word;
}

// Word w (0..7) of a tile's probabilities: the four keys 4w .. 4w+3 of the
// lane's 32 (S^T block w / 4, registers 4 (w % 4) ..), as P' = exp2(x) with
// x = s * coef + off, packed e4m3. Accumulates the fp32 sum and the max of x.
__device__ __forceinline__ uint32_t prob_word(const f32x16* s, int w, float coef, float off,
                                              float& l, float& mx) {
  const int b = w >> 2, r = (w & 3) * 4;
  const float x0 = fmaf(s[b][r], coef, off), x1 = fmaf(s[b][r + 1], coef, off);
  const float x2 = fmaf(s[b][r + 2], coef, off), x3 = fmaf(s[b][r + 3], coef, off);
  mx = fmaxf(fmaxf(mx, x0), fmaxf(x1, fmaxf(x2, x3)));
  float p0 = __builtin_amdgcn_exp2f(x0), p1 = __builtin_amdgcn_exp2f(x1);
  float p2 = __builtin_amdgcn_exp2f(x2), p3 = __builtin_amdgcn_exp2f(x3);
  uint32_t word = cvt_fp8x2<false>(p0, p1, 0u);
  word = cvt_fp8x2<true>(p2, p3, word);
  l += (p0 + p1) + (p2 + p3);
  // (keep the word and the sums in this slot: the instruction selector would
  // otherwise gather all softmax arithmetic at the end of the step)
  asm volatile("" : "+v"(word), "+v"(l), "+v"(mx));
  return word;
}

// S^T block of a tile from its K rows at kp (this lane's row, byte 32 g):
// two 64-dim steps, high and low query parts each, added to the seed c.
__device__ __forceinline__ f32x16 qk_block(const uint8_t* kp, const i32x8v* qf, const i32x8v* ql,
                                           const f32x16& c = f32x16{}) {
  const i32x8v k0 = lds_read32(kp), k1 = lds_read32(kp + 64);
  f32x16 s = mfma_fp8(k0, qf[0], c);
  s = mfma_fp8_blo(k0, ql[0], s);
  s = mfma_fp8(k1, qf[1], s);
  return mfma_fp8_blo(k1, ql[1], s);
}

// First part of a step (tile t), S^T of the tile in s (two 32-key blocks):
// PV of tile t-1 (P' in p_prev, V^T at vprev) and QK^T block 0 of tile t+1
// (K rows at kn0) on the matrix pipe, slot by slot beside the softmax of tile
// t into p_cur. Block 0 of s is consumed by words 0-3 and then receives block 0
// of tile t+1; block 1 still holds tile t. `boundary` runs after the first two
// MFMAs: it holds the barrier that makes K of tile t+1 visible. Returns the
// tile's fp32 sum of P'; mx gets the max of x over the row.
template <typename Boundary>
__device__ __forceinline__ float fp8_step_a(const uint8_t* vprev, const uint8_t* kn0,
                                            const i32x8v& p_prev, f32x16* o, const i32x8v* qf,
                                            const i32x8v* ql, f32x16* s, float coef, float off,
                                            i32x8v& p_cur, float& mx, Boundary&& boundary) {
  float l = 0.f;
  mx = -INFINITY;
  // slot 0: PV 0, 1; barrier; words 0, 1
  const i32x8v v0 = lds_read32(vprev), v1 = lds_read32(vprev + 32 * VS8);
  o[0] = mfma_fp8(v0, p_prev, o[0]);
  o[1] = mfma_fp8(v1, p_prev, o[1]);
  boundary();
  const i32x8v v2 = lds_read32(vprev + 64 * VS8), v3 = lds_read32(vprev + 96 * VS8);
  p_cur[0] = static_cast<int>(prob_word(s, 0, coef, off, l, mx));
  p_cur[1] = static_cast<int>(prob_word(s, 1, coef, off, l, mx));
  __builtin_amdgcn_sched_barrier(0);
  // slot 1: PV 2, 3; words 2, 3 (block 0 of tile t is then free)
  const i32x8v k0 = lds_read32(kn0), k1 = lds_read32(kn0 + 64);
  o[2] = mfma_fp8(v2, p_prev, o[2]);
  p_cur[2] = static_cast<int>(prob_word(s, 2, coef, off, l, mx));
  o[3] = mfma_fp8(v3, p_prev, o[3]);
  p_cur[3] = static_cast<int>(prob_word(s, 3, coef, off, l, mx));
  __builtin_amdgcn_sched_barrier(0);
  // slot 2: QK^T block 0 of tile t+1, first k-step; words 4, 5
  s[0] = mfma_fp8(k0, qf[0], f32x16{});
  p_cur[4] = static_cast<int>(prob_word(s, 4, coef, off, l, mx));
  s[0] = mfma_fp8_blo(k0, ql[0], s[0]);
  p_cur[5] = static_cast<int>(prob_word(s, 5, coef, off, l, mx));
  __builtin_amdgcn_sched_barrier(0);
  // slot 3: second k-step; words 6, 7
  s[0] = mfma_fp8(k1, qf[1], s[0]);
  p_cur[6] = static_cast<int>(prob_word(s, 6, coef, off, l, mx));
  s[0] = mfma_fp8_blo(k1, ql[1], s[0]);
  p_cur[7] = static_cast<int>(prob_word(s, 7, coef, off, l, mx));
  __builtin_amdgcn_sched_barrier(0);
  mx = max_other_half(mx);
  asm volatile("" : "+v"(p_cur), "+v"(l), "+v"(mx));
  return l;
}

// acc *= alpha, in place. Written as one asm block with every element tied to
// its register: as plain C++ in the rare rescale path, the register allocator
// keeps a second copy of the 64 output accumulators live and spills in the
// main loop. The compiler does not see hazards through inline asm, so the
// block waits out an MFMA still writing acc (leading nops) and lets the
// products settle before any MFMA reads them (trailing nops).
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
  float e[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = acc[r];
  asm volatile(
      "s_nop 7\n s_nop 7\n s_nop 7\n s_nop 7\n"
      "v_mul_f32 %0, %0, %16\n v_mul_f32 %1, %1, %16\n v_mul_f32 %2, %2, %16\n"
      "v_mul_f32 %3, %3, %16\n v_mul_f32 %4, %4, %16\n v_mul_f32 %5, %5, %16\n"
      "v_mul_f32 %6, %6, %16\n v_mul_f32 %7, %7, %16\n v_mul_f32 %8, %8, %16\n"
      "v_mul_f32 %9, %9, %16\n v_mul_f32 %10, %10, %16\n v_mul_f32 %11, %11, %16\n"
      "v_mul_f32 %12, %12, %16\n v_mul_f32 %13, %13, %16\n v_mul_f32 %14, %14, %16\n"
      "v_mul_f32 %15, %15, %16\n"
      "s_nop 7\n s_nop 7\n"
      : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]), "+v"(e[4]), "+v"(e[5]), "+v"(e[6]),
        "+v"(e[7]), "+v"(e[8]), "+v"(e[9]), "+v"(e[10]), "+v"(e[11]), "+v"(e[12]), "+v"(e[13]),
        "+v"(e[14]), "+v"(e[15])
      : "v"(alpha));
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = e[r];
}

// Rare path of a step, taken by the whole wave when some row's x exceeds
// kTrigger (P' would pass 362, near the e4m3 limit of 448): those rows move
// the running max up so that their largest x becomes kPTarget; O (every tile
// before this one) and the sum of the tiles before are scaled to match, and
// the tile's probabilities are recomputed -- block 0 of its S^T again from its
// K rows (kc0, still in LDS), block 1 from s1. Block 0 is masked like the
// first time, through the accumulator seed: -inf for keys past the count in
// `code` and for keys whose bit in wword is clear (all ones unless `code`
// flags a windowed text tile), 0 for the others.
__device__ __forceinline__ float rescale_step(float mx, float& m_run, float& off, float& l_run,
                                              f32x16* o, const uint8_t* kc0, const f32x16& s1,
                                              const i32x8v* qf, const i32x8v* ql, float coef,
                                              int code, int g, uint32_t wword, i32x8v& p_cur) {
  const float d = fmaxf(mx - kPTarget, 0.f);
  const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
  for (int i = 0; i < 4; ++i) scale_acc(o[i], alpha);
  l_run *= alpha;
  m_run += d;
  off -= d;
  float l = 0.f, m2 = -INFINITY;
  {
    f32x16 b0;
    const int lim = tile_count(code) - 32 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) b0[r] = r >= lim ? -INFINITY : keep_if_bit(0.f, wword, r);
    b0 = qk_block(kc0, qf, ql, b0);
#pragma unroll
    for (int w = 0; w < 4; ++w) p_cur[w] = static_cast<int>(prob_word_blk(b0, w, coef, off, l, m2));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) p_cur[4 + w] = static_cast<int>(prob_word_blk(s1, w, coef, off, l, m2));
  return l;
}

template <bool kSparse>
__global__ __launch_bounds__(kThreads, 1) void attn_fp8_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kStages * KT8];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kStages * VT8];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  __shared__ float red[kWaves];
  // timed-window bits (+ 1 word: lanes of group 1 on the last text tile may
  // read one word past the table; their keys are all masked by the valid count)
  __shared__ uint32_t wtab[kWindowWords + 1];
  __shared__ int woff[kThreads];

  const WorkTile wt = map_workgroup(a, BM);
  const AttnItemDev& I = a.items[wt.item];
  const int H = a.heads;
  const int h = wt.head;
  const int q0 = wt.q0;
  const int P = a.rope.P;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)

  const TileSeq seq = tile_seq(I, h, q0, BM, P);   // dense, or kept history blocks first
  int kt0, kt1;   // this work tile's logical key tiles
  key_range(a, I, P, wt.part, &kt0, &kt1);
  const int ntiles = kt1 - kt0;
  const int flag_fi = window_flag_segment(I);

  TileCursor lc;
  seq_start<kSparse, 1>(lc, I, h, H, P, seq, kt0);
  TileInfo ti0 = tile_info(lc, flag_fi);

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
  stage_window_table(I, wtab, q0, BM, P, tid, kThreads);
  // Every stage starts as zeros (the V stage of "tile -1" is read once with
  // zero probabilities; stages of tiles past the end may be read, unused).
  for (int i = tid; i < kStages * KT8 / 16; i += kThreads)
    reinterpret_cast<u32x4*>(Ks)[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < kStages * VT8 / 16; i += kThreads)
    reinterpret_cast<u32x4*>(Vs)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // Tiles load two ahead of the compute tile, K and then V (K of tile t+1 is
  // read in step t, V of tile t in step t+1). lc is the cursor of the last
  // tile loaded; ti0, ti1 carry tiles t, t+1.
  dma_k8(lc, Ks, w);
  dma_v8(lc, Vs, w);
  TileInfo ti1 = ti0;
  if (ntiles > 1) {
    seq_next<kSparse, 1>(lc, I, h, H, P, seq, kt0 + 1);
    ti1 = tile_info(lc, flag_fi);
    dma_k8(lc, Ks + KT8, w);
    dma_v8(lc, Vs + VT8, w);
  }
  vmax = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) vmax = fmaxf(vmax, red[i]);

  // ---- Q: rotate in fp32, quantise per (row, head) to e4m3 ---------------------
  // lane holds dims 64*kk + 32*g + e (kk = 0, 1; e = 0..31) of its query row.
  // The query is split: qf = e4m3(q * 448 / amax), ql = e4m3(16 * residual), so
  // that qf + ql / 16 carries about 7 significant bits instead of 4.
  const int qrow = q0 + 32 * w + r32;
  // This lane's window word for key tile kt0 + tt (a text tile under
  // windows): bits of keys 32 g .. 32 g + 31. Each thread's table offset waits
  // in LDS (woff, read back only by the same thread) and is found from the
  // lane index on each use, which keeps it out of the loop's registers.
  woff[tid] = window_row_offset(I, q0, qrow, P) + g;
  auto window_word = [&](int tt) __attribute__((always_inline)) {
    const int t = static_cast<int>(lane_here()) + 64 * w;
    return wtab[woff[t] + (max(text_tile_base(I, P, kt0 + tt), 0) >> 5)];
  };
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

  // tiles 0 and 1 are in LDS before the first step
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
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

  // S^T of tile 0; the running max m (log2 units) starts at its max
  f32x16 sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) sc[b] = qk_block(Ks + krow[b] * KS8 + 32 * g, qf, ql);
  if (ti0.nvalid < BN) mask_tile(sc, tile_count(ti0.nvalid), g);
  // (tile 0 is never a text tile under timed windows: the key ranges of such
  // items start on a video tile, so every row sees tile 0's valid keys)
  float m_run;
  {
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][r]);
    m_run = max_other_half(mx) * (c2 * ti0.kscale);   // tile 0 always has a valid key
  }
  i32x8v pa = {}, pb;
  const float pf_base = kPScale / vmax;

  // Tile t sits in stage t % 4. Step t: PV(t-1) and QK^T(t+1) on the matrix
  // pipe beside the softmax of tile t; S^T is computed in place (block 0 of
  // tile t+1 after words 0-3 of tile t, block 1 after the rescale check). The
  // barrier of step t comes after its first two (PV) MFMAs; K of tile t+1
  // (loaded in step t-1) is read after it. Two steps per loop trip: the P
  // buffers swap roles without copies.
  int pending = 0;   // lower bound of this wave's loads issued in the step before
  auto step = [&](int tt, const i32x8v& p_prev, i32x8v& p_cur) __attribute__((always_inline)) {
    const uint8_t* Vprev = Vs + ((tt + kStages - 1) & (kStages - 1)) * VT8 + voff;
    const uint8_t* Kcur = Ks + (tt & (kStages - 1)) * KT8 + 32 * g;
    const uint8_t* Knext = Ks + ((tt + 1) & (kStages - 1)) * KT8 + 32 * g;
    const TileInfo cur = ti0;
    TileInfo ti2 = ti0;
    // Before the barrier each wave waits for its K load of the step before
    // (tile t+1, read in this step); its V load (read two steps later) stays in
    // flight. After the barrier, tile t+2 goes into stage (t+2) % 4, the stage
    // of tile t-2 (its V was last read in step t-1, its K in step t-3).
    auto boundary = [&]() __attribute__((always_inline)) {
      wait_loads(pending);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      pending = 0;
      if (tt + 2 < ntiles) {
        const int s2 = (tt + 2) & (kStages - 1);
        seq_next<kSparse, 1>(lc, I, h, H, P, seq, kt0 + tt + 2);
        ti2 = tile_info(lc, flag_fi);
        dma_k8(lc, Ks + s2 * KT8, w);
        dma_v8(lc, Vs + s2 * VT8, w);
        pending = 1;   // every wave issues at least one V load
      }
    };
    if (cur.nvalid < BN) {   // partial tile, or text tile with windows
      if (tile_count(cur.nvalid) < BN) mask_tile(sc, tile_count(cur.nvalid), g);
      if (cur.nvalid < 0) window_mask_tile(sc, window_word(tt));
    }
    const float coef = c2 * cur.kscale;
    const float pf = pf_base * cur.vscale;
    float off8 = __log2f(pf) - m_run;
    float mx;
    float lt = fp8_step_a(Vprev, Knext + krow[0] * KS8, p_prev, o, qf, ql, sc, coef, off8, p_cur,
                          mx, boundary);
    if (__builtin_expect(__any(mx > kTrigger), 0))
      lt = rescale_step(mx, m_run, off8, l_run, o, Kcur + krow[0] * KS8, sc[1], qf, ql, coef,
                        cur.nvalid, g, cur.nvalid < 0 ? window_word(tt) : ~0u, p_cur);
    // QK^T block 1 of tile t+1 (block 1 of tile t is no longer needed)
    sc[1] = qk_block(Knext + krow[1] * KS8, qf, ql);
    l_run += lt / pf;
    ti0 = ti1;
    ti1 = ti2;
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
  if (wt.part >= 0) {   // split tile: partial result for the merge kernel
    if (qrow < I.n_q)
      store_partial(a, wt.unit, BM, qrow - q0, g, o, vmax / kPScale, m_run, l_tot);
    return;
  }
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
  if (a.any_sparse)
    hipLaunchKernelGGL(attn_fp8_kernel<true>, dim3(a.grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fp8_kernel<false>, dim3(a.grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
