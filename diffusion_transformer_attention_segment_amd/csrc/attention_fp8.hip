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
// plane (per head for the text slot), a power of two 2^e (sa_kv_append writes
// such scales). A key tile never straddles a frame, so its K and V scales are
// uniform over the tile, and the fp32 exponent field of a scale is exactly the
// E8M0 block scale (127 + e) of the fp8 MFMA: the K scale enters Q.K^T and the
// V scale enters P.V through the A operand's block scale, exactly.
// Queries are rotated in fp32 and multiplied by softmax scale * log2(e), then
// quantised per (row, head) with a power-of-two scale 2^qe (amax <= 448 * 2^qe)
// in two parts: y = q * 2^-qe, hi = e4m3(y), lo = e4m3(16 (y - hi)),
// q ~ (hi + lo / 16) 2^qe. Both parts enter through the B operand's block
// scales (127 + qe and 127 + qe - 4, two bytes of one register), so the QK^T
// accumulator holds the logit in log2 units. It starts from 6 - m (m the
// running max), so a probability is P'_j = exp2(acc_j) = 2^6 p_j, one exp2
// per key (the 2^6 keeps small probabilities out of the e4m3 subnormal
// range); O = sum_j P'_j v_j and l = sum_j P'_j, out = O / l. The running
// max m moves (rarely) when the sum of some lane's four consecutive P'
// passes 2^8.5 = 362, to put the largest acc at 6. Such a sum is computed
// for l anyway, so the overflow guard costs one max per eight keys: while no
// sum passes 362 no P' does (e4m3 max 448), and a sum passes it only if some
// P' passes 2^6.5, i.e. some acc passes 6.5.
// Q is never stored, so its split costs only a second MFMA per k-step and
// removes most of the query's share of the fp8 error; the cache keeps one
// e4m3 code per value.
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
// 4-stage ring, one barrier per tile. With block-sparse history, the kept
// tiles' plane offsets and scales are staged in LDS before the key loop, so a
// jump to the next kept tile reads no memory on the scalar path.
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
constexpr float kPTarget = 6.0f;       // log2 of P' for the largest key (probabilities x 2^6)
constexpr float kTriggerSum = 362.03867f;   // 2^8.5: a lane's sum of four P' above it moves
                                            // the running max
constexpr int kMaxShift = 64;          // largest shift of the running max carried by the
                                       // P.V block scale before O is renormalised

typedef int i32x8v __attribute__((ext_vector_type(8)));

// e4m3 x e4m3 MFMA with E8M0 block scales: A scaled by 2^(sa - 127), B by
// 2^(byte 0 of sb - 127) (mfma_fp8) or 2^(byte 1 of sb - 127) (mfma_fp8_b1).
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8v& a, const i32x8v& b, const f32x16& c,
                                           int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x16 mfma_fp8_b1(const i32x8v& a, const i32x8v& b, const f32x16& c,
                                              int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 1, sb);
}

constexpr int kUnitScale = 127;   // E8M0 2^0

// E8M0 block scale of a power-of-two fp32 scale: its exponent field
__device__ __forceinline__ int e8m0_of(float pow2_scale) {
  return static_cast<int>((__float_as_uint(pow2_scale) >> 23) & 0xFFu);
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
// slots (64 data bytes + pad). Load j of a stage fills its slots 64 j ..
// 64 j + 63 (dma_tile); wave w issues loads w and w + 8 (the second only where
// it exists: K has 9 loads, V^T 10). A lane's global offsets for them depend
// only on the row length, so they are computed once: for K rows (128 bytes)
// and for V^T rows of a frame plane (PL bytes, its token slots); the text
// slot's V^T rows (text capacity bytes) take dma_tile's per-tile computation.
constexpr int kKLoads = BN * (KS8 / 16) / 64;    // 9
constexpr int kVLoads = kD * (VS8 / 16) / 64;    // 10

struct DmaOffsets {
  uint32_t k[2];
  uint32_t v[2];
};

__device__ __forceinline__ uint32_t slot_offset(uint32_t n, uint32_t slots, uint32_t row_bytes) {
  const uint32_t row = n / slots, ch = n - slots * row;
  return ch == slots - 1 ? kOutOfRange : row * row_bytes + ch * 16u;
}

__device__ __forceinline__ DmaOffsets dma_offsets(int w, int lane, int v_row_bytes) {
  DmaOffsets d;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t n = 64u * (w + 8 * m) + lane;
    d.k[m] = slot_offset(n, KS8 / 16, kD);
    d.v[m] = slot_offset(n, VS8 / 16, static_cast<uint32_t>(v_row_bytes));
  }
  return d;
}

__device__ __forceinline__ void dma_k8(const TileCursor& c, uint8_t* stage, int w,
                                       const DmaOffsets& d) {
  const __amdgpu_buffer_rsrc_t r = tile_k_rsrc<1>(c);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int j = w + 8 * m;
    if (j < kKLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(stage + 1024 * j), 16, d.k[m], 0, 0, 0);
  }
}

__device__ __forceinline__ void dma_v8(const TileCursor& c, uint8_t* stage, int w, int PL,
                                       const DmaOffsets& d) {
  if (c.vstride != PL) {   // the text slot
    dma_tile<kD, VS8 / 16>(tile_v_rsrc<1>(c), stage, static_cast<uint32_t>(c.vstride), w);
    return;
  }
  const __amdgpu_buffer_rsrc_t r = tile_v_rsrc<1>(c);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int j = w + 8 * m;
    if (j < kVLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(stage + 1024 * j), 16, d.v[m], 0, 0, 0);
  }
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
  int ksc;      // E8M0 block scales of the tile's K and V planes
  int vsc;
};

__device__ __forceinline__ TileInfo tile_info(const TileCursor& c, int flag_fi) {
  TileInfo t;
  t.nvalid = cursor_mask_code(c, flag_fi);
  t.ksc = e8m0_of(c.kscale);
  t.vsc = e8m0_of(c.vscale);
  return t;
}

// Block-sparse history: the kept tiles of a work tile are staged in LDS before
// the key loop, one 16-byte entry per tile: the byte offset of the tile's
// (frame, head) plane in the K and V caches (64 bits), and the tile's index in
// its frame with the E8M0 bytes of the plane's K and V scales. A jump to a
// kept tile then reads LDS instead of the chain of dependent scalar loads
// (list entry, frame entry, plane scales) that would stall the wave.
constexpr int kKeptTab = 4096;   // entries; later kept tiles take the scalar walk

__device__ __forceinline__ void cursor_kept(TileCursor& c, const char* kbase, const char* vbase,
                                            uint32_t off_lo, uint32_t off_hi, uint32_t w1, int P,
                                            int PL) {
  const size_t plane = (static_cast<size_t>(off_hi) << 32) | off_lo;
  c.fi = 0;   // a history frame: never a text segment under timed windows
  c.p0 = static_cast<int>(w1 & 0xFFFFu) * kKeyTile;
  c.len = P;
  c.vstride = PL;
  c.kplane = kbase + plane;
  c.vplane = vbase + plane;
  c.kscale = __uint_as_float(((w1 >> 16) & 0xFFu) << 23);
  c.vscale = __uint_as_float((w1 >> 24) << 23);
}

// Word w (0..3) of one 32-key block: keys 4w .. 4w+3 of the block (registers
// 4w ..), as P' = exp2(acc) packed e4m3. Accumulates the fp32 sum of P'.
__device__ __forceinline__ uint32_t prob_word_blk(const f32x16& s, int w, float& l) {
  const int r = w * 4;
  const float p0 = __builtin_amdgcn_exp2f(s[r]), p1 = __builtin_amdgcn_exp2f(s[r + 1]);
  const float p2 = __builtin_amdgcn_exp2f(s[r + 2]), p3 = __builtin_amdgcn_exp2f(s[r + 3]);
  uint32_t word = cvt_fp8x2<false>(p0, p1, 0u);
  word = cvt_fp8x2<true>(p2, p3, word);
  l += (p0 + p1) + (p2 + p3);
  return word;
}

// Word w (0..7) of a tile's probabilities: the four keys 4w .. 4w+3 of the
// lane's 32 (S^T block w / 4, registers 4 (w % 4) ..), as P' = exp2(acc)
// packed e4m3, built in place of `old` (the register's previous word, so that
// no zero is written first). q gets the four keys' sum of P', which is added
// to l.
__device__ __forceinline__ uint32_t prob_word(const f32x16* s, int w, float& l, float& q,
                                              uint32_t old) {
  const int b = w >> 2, r = (w & 3) * 4;
  float p0 = __builtin_amdgcn_exp2f(s[b][r]), p1 = __builtin_amdgcn_exp2f(s[b][r + 1]);
  float p2 = __builtin_amdgcn_exp2f(s[b][r + 2]), p3 = __builtin_amdgcn_exp2f(s[b][r + 3]);
  uint32_t word = cvt_fp8x2<false>(p0, p1, old);
  word = cvt_fp8x2<true>(p2, p3, word);
  q = (p0 + p1) + (p2 + p3);
  l += q;
  // (keep the word and the sums in this slot: the instruction selector would
  // otherwise gather all softmax arithmetic at the end of the step)
  asm volatile("" : "+v"(word), "+v"(l), "+v"(q));
  return word;
}

// The accumulator seed: 16 copies of this lane's 6 - m. It is built once and
// stays live across the key loop (moved only by a rescale), so every QK^T
// block reads it as its accumulator input with no copies on the common path.
__device__ __forceinline__ f32x16 splat_seed(float pseed) {
  // a register pair holding the value twice, then seven 64-bit copies of it.
  // The compiler does not see hazards inside inline asm: the trailing nops
  // give an MFMA that reads the copies as its accumulator the wait states a
  // VALU write needs before that read.
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  f32x2v pair = {pseed, pseed};
  asm volatile("" : "+v"(pair));
  f32x2v c1, c2, c3, c4, c5, c6, c7;
  asm volatile(
      "v_mov_b64 %0, %7\n v_mov_b64 %1, %7\n v_mov_b64 %2, %7\n v_mov_b64 %3, %7\n"
      "v_mov_b64 %4, %7\n v_mov_b64 %5, %7\n v_mov_b64 %6, %7\n s_nop 4"
      : "=v"(c1), "=v"(c2), "=v"(c3), "=v"(c4), "=v"(c5), "=v"(c6), "=v"(c7)
      : "v"(pair));
  const f32x2v parts[8] = {pair, c1, c2, c3, c4, c5, c6, c7};
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    c[2 * r] = parts[r][0];
    c[2 * r + 1] = parts[r][1];
  }
  return c;
}

// S^T block of a tile from its K rows at kp (this lane's row, byte 32 g):
// two 64-dim steps, high and low query parts each (block scales: the tile's
// K scale ksc; qsc holds the query's high and low part scales), added to the
// seed c.
__device__ __forceinline__ f32x16 qk_block(const uint8_t* kp, const i32x8v* qf, const i32x8v* ql,
                                           int ksc, int qsc, const f32x16& c) {
  const i32x8v k0 = lds_read32(kp), k1 = lds_read32(kp + 64);
  f32x16 s = mfma_fp8(k0, qf[0], c, ksc, qsc);
  s = mfma_fp8_b1(k0, ql[0], s, ksc, qsc);
  s = mfma_fp8(k1, qf[1], s, ksc, qsc);
  return mfma_fp8_b1(k1, ql[1], s, ksc, qsc);
}

// First part of a step (tile t), S^T of the tile in s (two 32-key blocks):
// PV of tile t-1 (P' in p_prev, V^T at vprev) and QK^T block 0 of tile t+1
// (K rows at kn0) on the matrix pipe, slot by slot beside the softmax of tile
// t into p_cur. Block 0 of s is consumed by words 0-3 and then receives block 0
// of tile t+1; block 1 still holds tile t. `boundary` runs after the first two
// MFMAs: it holds the barrier that makes K of tile t+1 visible. Returns the
// tile's fp32 sum of P' (this lane's 32 keys); mx gets the largest of the
// lane's eight 4-key sums of P'.
template <typename Boundary>
__device__ __forceinline__ float fp8_step_a(const uint8_t* vprev, const uint8_t* kn0,
                                            const i32x8v& p_prev, int vsc_prev, int psc, f32x16* o,
                                            const i32x8v* qf, const i32x8v* ql, int ksc_next,
                                            int qsc, const f32x16& seed, f32x16* s,
                                            i32x8v& p_cur, float& mx, Boundary&& boundary) {
  float l = 0.f, qa, qb;
  mx = 0.f;
  // slot 0: PV 0, 1; barrier; words 0, 1
  const i32x8v v0 = lds_read32(vprev), v1 = lds_read32(vprev + 32 * VS8);
  o[0] = mfma_fp8(v0, p_prev, o[0], vsc_prev, psc);
  o[1] = mfma_fp8(v1, p_prev, o[1], vsc_prev, psc);
  boundary();
  const i32x8v v2 = lds_read32(vprev + 64 * VS8), v3 = lds_read32(vprev + 96 * VS8);
  p_cur[0] = static_cast<int>(prob_word(s, 0, l, qa, static_cast<uint32_t>(p_cur[0])));
  p_cur[1] = static_cast<int>(prob_word(s, 1, l, qb, static_cast<uint32_t>(p_cur[1])));
  mx = fmaxf(fmaxf(mx, qa), qb);
  __builtin_amdgcn_sched_barrier(0);
  // slot 1: PV 2, 3; words 2, 3 (block 0 of tile t is then free)
  const i32x8v k0 = lds_read32(kn0), k1 = lds_read32(kn0 + 64);
  o[2] = mfma_fp8(v2, p_prev, o[2], vsc_prev, psc);
  p_cur[2] = static_cast<int>(prob_word(s, 2, l, qa, static_cast<uint32_t>(p_cur[2])));
  o[3] = mfma_fp8(v3, p_prev, o[3], vsc_prev, psc);
  p_cur[3] = static_cast<int>(prob_word(s, 3, l, qb, static_cast<uint32_t>(p_cur[3])));
  mx = fmaxf(fmaxf(mx, qa), qb);
  __builtin_amdgcn_sched_barrier(0);
  // slot 2: QK^T block 0 of tile t+1, first k-step (from the seed 6 - m);
  // words 4, 5
  s[0] = mfma_fp8(k0, qf[0], seed, ksc_next, qsc);
  p_cur[4] = static_cast<int>(prob_word(s, 4, l, qa, static_cast<uint32_t>(p_cur[4])));
  s[0] = mfma_fp8_b1(k0, ql[0], s[0], ksc_next, qsc);
  p_cur[5] = static_cast<int>(prob_word(s, 5, l, qb, static_cast<uint32_t>(p_cur[5])));
  mx = fmaxf(fmaxf(mx, qa), qb);
  __builtin_amdgcn_sched_barrier(0);
  // slot 3: second k-step; words 6, 7
  s[0] = mfma_fp8(k1, qf[1], s[0], ksc_next, qsc);
  p_cur[6] = static_cast<int>(prob_word(s, 6, l, qa, static_cast<uint32_t>(p_cur[6])));
  s[0] = mfma_fp8_b1(k1, ql[1], s[0], ksc_next, qsc);
  p_cur[7] = static_cast<int>(prob_word(s, 7, l, qb, static_cast<uint32_t>(p_cur[7])));
  mx = fmaxf(fmaxf(mx, qa), qb);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" : "+v"(p_cur), "+v"(l), "+v"(mx));
  return l;
}

// Rare path of a step, taken by the whole wave when some lane's 4-key sum of
// P' passes kTriggerSum (a P' near the e4m3 limit of 448 is possible): rows
// whose largest acc in the tile passes kPTarget move the running max up so
// that it becomes kPTarget. The tile's acc is found again for that -- block 0
// of its S^T from its K rows (kc0, still in LDS; block scale ksc) with the old
// seed, block 1 in s[1]. O (every tile before this one), the sum of the tiles
// before, the seed and block 0 of the next tile (already issued from the old
// seed) are shifted to match, and the tile's probabilities are recomputed.
// Block 0 is masked like the first time, through the accumulator seed: -inf
// for keys past the count in `code` and for keys whose bit in wword is clear
// (all ones unless `code` flags a windowed text tile).
__device__ __forceinline__ float rescale_step(float& l_run, int& shift,
                                              float& pseed, f32x16& seed, f32x16* s,
                                              const uint8_t* kc0,
                                              const i32x8v* qf, const i32x8v* ql, int ksc, int qsc,
                                              int code, int g, uint32_t wword, i32x8v& p_cur) {
  // an integer shift d: O keeps the units of the max before all shifts, and the
  // later probabilities enter P.V with the block scale 2^shift
  f32x16 b0;
  {
    const int lim = tile_count(code) - 32 * g;
#pragma unroll
    for (int r = 0; r < 16; ++r) b0[r] = (r >= lim ? -INFINITY : keep_if_bit(0.f, wword, r)) + pseed;
    b0 = qk_block(kc0, qf, ql, ksc, qsc, b0);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, b0[r]), s[1][r]);
  mx = max_other_half(mx);
  const float d = fmaxf(ceilf(mx - kPTarget), 0.f);
  l_run *= __builtin_amdgcn_exp2f(-d);
  shift += static_cast<int>(d);
  // whole-vector updates, so that each value keeps its registers across the
  // branch (element-wise updates leave copies on the common path)
  pseed -= d;
  seed = seed - d;
  s[0] = s[0] - d;
  b0 = b0 - d;
  float l = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) p_cur[w] = static_cast<int>(prob_word_blk(b0, w, l));
  const f32x16 b1 = s[1] - d;
#pragma unroll
  for (int w = 0; w < 4; ++w) p_cur[4 + w] = static_cast<int>(prob_word_blk(b1, w, l));
  return l;
}

template <bool kSparse>
__global__ __launch_bounds__(kThreads, 1) void attn_fp8_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kStages * KT8];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kStages * VT8];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  // timed-window bits (+ 1 word: lanes of group 1 on the last text tile may
  // read one word past the table; their keys are all masked by the valid count)
  __shared__ uint32_t wtab[kWindowWords + 1];
  __shared__ int woff[kThreads];
  __shared__ uint4 ktab[kSparse ? kKeptTab : 1];   // kept tiles of the work tile

  const WorkTile wt = map_workgroup(a, BM);
  const AttnItemDev& I = a.items[wt.item];
  const int H = a.heads;
  const int h = wt.head;
  const int q0 = wt.q0;
  const int P = a.rope.P;
  const int PL = plane_tokens(P, true);   // token slots (V^T row bytes) of a frame plane
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

  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  stage_window_table(I, wtab, q0, BM, P, tid, kThreads);
  int n_tab = 0;   // kept tiles staged (logical tiles kt0 .. kt0 + n_tab - 1)
  if constexpr (kSparse) {
    const int tpf = (P + kKeyTile - 1) / kKeyTile;
    // (an entry holds the tile's index in its frame in 16 bits)
    n_tab = tpf <= 0x10000 ? min(max(0, min(kt1, seq.keep) - kt0), kKeptTab) : 0;
    for (int i = tid; i < n_tab; i += kThreads) {
      const int tile = seq.list[kt0 + i];
      const int fi = tile / tpf;
      const int frame = I.frames[fi];
      const size_t pl = static_cast<size_t>(frame) * H + h;
      const size_t off = pl * static_cast<size_t>(PL) * kD;
      const uint32_t ks = static_cast<uint32_t>(e8m0_of(I.k_scale[pl]));
      const uint32_t vs = static_cast<uint32_t>(e8m0_of(I.v_scale[pl]));
      ktab[i] = make_uint4(static_cast<uint32_t>(off), static_cast<uint32_t>(off >> 32),
                           static_cast<uint32_t>(tile - fi * tpf) | (ks << 16) | (vs << 24), 0u);
    }
  }
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
  const DmaOffsets dmo = dma_offsets(w, lane, PL);
  dma_k8(lc, Ks, w, dmo);
  dma_v8(lc, Vs, w, PL, dmo);
  TileInfo ti1 = ti0;
  if (ntiles > 1) {
    seq_next<kSparse, 1>(lc, I, h, H, P, seq, kt0 + 1);
    ti1 = tile_info(lc, flag_fi);
    dma_k8(lc, Ks + KT8, w, dmo);
    dma_v8(lc, Vs + VT8, w, PL, dmo);
  }
  // ---- Q: rotate in fp32, times softmax scale * log2(e), quantise per (row,
  // head) to e4m3 -----------------------------------------------------------------
  // lane holds dims 64*kk + 32*g + e (kk = 0, 1; e = 0..31) of its query row.
  // The query is split: qf = e4m3(q * 2^-qe), ql = e4m3(16 * residual), so
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
  int qsc;   // E8M0 block scales of the high (byte 0) and low (byte 1) parts
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
          x[32 * kk + 8 * ch + 2 * m] = xa * a.scale_log2;
          x[32 * kk + 8 * ch + 2 * m + 1] = xb * a.scale_log2;
        }
      }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = max_other_half(amax);
    // 2^qe: the least power of two with amax <= 448 * 2^qe (448 = 1.75 * 2^8),
    // at least 2^-122 so that the low part's scale 2^(qe - 4) stays an E8M0
    // value; 2^0 for a zero row
    int qe = 0;
    if (amax > 0.f) {
      const uint32_t b = __float_as_uint(amax);
      qe = static_cast<int>(b >> 23) - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
      qe = max(qe, -122);
    }
    const float inv = __uint_as_float(static_cast<uint32_t>(127 - qe) << 23);   // 2^-qe
    qsc = (127 + qe) | ((123 + qe) << 8);
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
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float l_run = 0.f;

  // S^T of tile 0 (logits in log2 units); the running max m starts at its max,
  // and every later QK^T accumulation starts from the seed 6 - m
  f32x16 sc[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) sc[b] = qk_block(Ks + krow[b] * KS8 + 32 * g, qf, ql, ti0.ksc, qsc, f32x16{});
  if (ti0.nvalid < BN) mask_tile(sc, tile_count(ti0.nvalid), g);
  // (tile 0 is never a text tile under timed windows: the key ranges of such
  // items start on a video tile, so every row sees tile 0's valid keys)
  // The running max is m_ref + shift: probabilities P' = 2^(x - m_ref - shift + 6)
  // enter P.V with the block scale 2^shift, so O stays in units of 2^(x - m_ref
  // + 6) and a rescale never rewrites it; l_run is in the units of the running
  // max. O is renormalised (m_ref moves up) only when a shift passes kMaxShift.
  float m_ref;
  {
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[b][r]);
    m_ref = max_other_half(mx);   // tile 0 always has a valid key
  }
  int shift = 0;
  uint32_t n_resc = 0, n_renorm = 0;   // this wave's rescales (diagnostic counters only)
  float pseed = kPTarget - m_ref;   // the seed of every later QK^T accumulation
#pragma unroll
  for (int b = 0; b < 2; ++b) sc[b] = sc[b] + pseed;
  i32x8v pa = {}, pb = {};
  f32x16 seed = splat_seed(pseed);   // the accumulator seed of every QK^T block
  int vsc_prev = kUnitScale;   // V block scale of the tile before the compute tile

  // Tile t sits in stage t % 4. Step t: PV(t-1) and QK^T(t+1) on the matrix
  // pipe beside the softmax of tile t; S^T is computed in place (block 0 of
  // tile t+1 after words 0-3 of tile t, block 1 after the rescale check). The
  // barrier of step t comes after its first two (PV) MFMAs; K of tile t+1
  // (loaded in step t-1) is read after it. Two steps per loop trip: the P
  // buffers swap roles without copies.
  // The key walk's next tile: a staged kept tile (its entry read from LDS one
  // step ahead, into ent), else the scalar walk.
  const char* kbase = static_cast<const char*>(I.k);
  const char* vbase = static_cast<const char*>(I.v);
  uint4 ent = make_uint4(0u, 0u, 0u, 0u);   // entry of the kept tile the next advance takes
  if constexpr (kSparse) {
    if (n_tab > 2) ent = ktab[2];
  }
  auto advance = [&](int li) __attribute__((always_inline)) {
    if constexpr (kSparse) {
      const int i = li - kt0;   // >= 2: tiles kt0 and kt0 + 1 are loaded before the loop
      if (i < n_tab) {
        const uint32_t off_lo = __builtin_amdgcn_readfirstlane(ent.x);
        const uint32_t off_hi = __builtin_amdgcn_readfirstlane(ent.y);
        const uint32_t w1 = __builtin_amdgcn_readfirstlane(ent.z);
        if (i + 1 < n_tab) ent = ktab[i + 1];
        cursor_kept(lc, kbase, vbase, off_lo, off_hi, w1, P, PL);
        return;
      }
    }
    seq_next<kSparse, 1>(lc, I, h, H, P, seq, li);
  };
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
        advance(kt0 + tt + 2);
        ti2 = tile_info(lc, flag_fi);
        dma_k8(lc, Ks + s2 * KT8, w, dmo);
        dma_v8(lc, Vs + s2 * VT8, w, PL, dmo);
        pending = 1;   // every wave issues at least one V load
      }
    };
    if (cur.nvalid < BN) {   // partial tile, or text tile with windows
      if (tile_count(cur.nvalid) < BN) mask_tile(sc, tile_count(cur.nvalid), g);
      if (cur.nvalid < 0) window_mask_tile(sc, window_word(tt));
    }
    const int ksc_next = ti1.ksc;
    float mx;
    float lt = fp8_step_a(Vprev, Knext + krow[0] * KS8, p_prev, vsc_prev, kUnitScale + shift, o, qf,
                          ql, ksc_next, qsc, seed, sc, p_cur, mx, boundary);
    if (__builtin_expect(__any(mx > kTriggerSum), 0)) {
      lt = rescale_step(l_run, shift, pseed, seed, sc, Kcur + krow[0] * KS8, qf, ql, cur.ksc, qsc,
                        cur.nvalid, g, cur.nvalid < 0 ? window_word(tt) : ~0u, p_cur);
      ++n_resc;
    }
    // QK^T block 1 of tile t+1 (block 1 of tile t is no longer needed)
    sc[1] = qk_block(Knext + krow[1] * KS8, qf, ql, ksc_next, qsc, seed);
    l_run += lt;
    vsc_prev = cur.vsc;
    ti0 = ti1;
    ti1 = ti2;
  };
  // A step whose rescale leaves a shift above kMaxShift stops the loop before
  // the next step's P.V, which would take block scale 127 + shift: O is
  // renormalised here, off the loop's path, and the loop resumes. (Stopping
  // after the first of a trip's two steps, the probabilities of that step move
  // into pa so that the resumed trip starts with them.)
  int t = 0;
  int base = 0;     // the step the last (re)started loop began with
  for (;;) {
    int stop = 0;   // 1: after a trip's first step, 2: after its second
#pragma unroll 1
    for (; t < ntiles; t += 2) {
      step(t, pa, pb);
      if (__builtin_expect(__any(shift > kMaxShift), 0)) {
        stop = 1;
        break;
      }
      if (t + 1 < ntiles) {
        step(t + 1, pb, pa);
        if (__builtin_expect(__any(shift > kMaxShift), 0)) {
          stop = 2;
          break;
        }
      }
    }
    if (stop == 0) break;
    ++n_renorm;
    const float alpha = __builtin_amdgcn_exp2f(-static_cast<float>(shift));
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = o[i] * alpha;
    m_ref += static_cast<float>(shift);
    shift = 0;
    if (stop == 1) {
      pa = pb;
      t += 1;
    } else {
      t += 2;
    }
    base = t;
  }
  {
    const uint8_t* Vlast = Vs + ((ntiles - 1) & (kStages - 1)) * VT8;
    // trips from `base` write pb, then pa: an odd count of steps ends in pb
    const i32x8v& p_last = ((ntiles - base) & 1) ? pb : pa;
#pragma unroll
    for (int db = 0; db < 4; ++db)
      o[db] = mfma_fp8(lds_read32(Vlast + voff + 32 * db * VS8), p_last, o[db], vsc_prev,
                       kUnitScale + shift);
  }

  // The output MFMAs compute across all lanes of the wave: keep them (and
  // everything feeding them) ahead of the per-row store branch below, where
  // lanes past the last query row are switched off.
  asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));

  if (a.counters != nullptr) add_counts(a.counters, tid, n_renorm, n_resc);

  // ---- epilogue ----------------------------------------------------------------
  // O and l in units of 2^(x - m_ref + 6): m_ref - 6 is the max the merge sees
  const float l_tot = (l_run + __shfl_xor(l_run, 32)) *
                      __uint_as_float(static_cast<uint32_t>(127 + shift) << 23);   // x 2^shift
  const float inv = 1.0f / l_tot;
  if (wt.part >= 0) {   // split tile: partial result for the merge kernel
    if (qrow < I.n_q)
      store_partial(a, wt.unit, BM, qrow - q0, g, o, 1.0f, m_ref - kPTarget, l_tot);
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
      I.lse[static_cast<size_t>(qrow) * H + h] =
          (m_ref - kPTarget + __log2f(l_tot)) * 0.6931471805599453f;
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
