// segment_attention, bf16 cache: fused Q-RoPE + flash-style attention over a
// gathered key set (kept history frames via an index list, the current
// segment's frames, the text slot), bf16 MFMA on gfx950, fp32 accumulation.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// sections "How one segment is made" (joint attention of the segment's video
// and text tokens, 16 heads of 128, 3D RoPE, reading history from a KV cache)
// and "The 4090 preset" (a picked subset of past frames is attended).
//
// Work decomposition. One workgroup = 8 waves = 256 query rows of one head of
// one session (two waves per SIMD); each wave owns 32 rows. Key tiles of 64
// keys never straddle a frame (a frame of P tokens is ceil(P/64) tiles), so a
// tile is one frame-plane base plus a row offset: tiles are fetched with
// buffer loads whose resource bounds zero-fill the rows past the frame end,
// and the frame list is read once per frame by a scalar cursor. K/V tiles go
// HBM -> registers -> a 4-stage LDS ring (one barrier per tile); the loads of
// tile t+3 are in flight while tile t is computed.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, 32x32 output, K = 16):
//   S^T = K . Q^T   A = K rows (keys), B = Q^T (queries = lanes % 32)
//   O^T = V^T . P^T A = V^T rows (dims), B = P^T (queries = lanes % 32)
// The S^T accumulator of lane l holds, for query l % 32, A rows
// 8*(r/4) + 4*(l/32) + r%4 (register r). Loading K row pi(r) = r with bits 2
// and 3 swapped into A row r makes lane-group g hold the contiguous keys
// 16c + 8g .. 16c + 8g + 7 in registers 8c .. 8c + 7, exactly the B-operand
// layout P^T needs -- so P never leaves registers, and V^T (stored transposed
// in the cache) is read from LDS as contiguous 16 bytes.
//
// In-wave pipeline over 32-key blocks: step j issues, in one basic block,
// PV of block j-1 and QK^T of block j+1 (alternating, so the dependent QK^T
// chain is interleaved with independent PV work) next to the softmax VALU work
// of block j (its max and its exponentials against the running max). When the
// block max exceeds the running max by more than the slack -- rare after the
// first blocks -- a wave-uniform branch rescales O and the sum and recomputes
// the block's probabilities.
#include <type_traits>

#include "attention_common.h"

namespace segattn {
namespace {

constexpr int BM = 256;          // query rows per workgroup
static_assert(BM == SA_SPARSE_QUERY_BLOCK, "a work tile reads one block list");
constexpr int BN = kKeyTile;     // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;       // LDS ring depth (power of two)
constexpr int KS = kD + 8;       // LDS row stride of the K tile (elements): 272 B
constexpr int VS = BN + 8;       // LDS row stride of the V^T tile (elements): 144 B
constexpr int KT = BN * KS;      // elements of one K stage
constexpr int VT = kD * VS;      // elements of one V^T stage
constexpr int kKChunks = BN * kD / 8 / kThreads;   // 16-byte K chunks per thread (2)
constexpr int kVChunks = kD * BN / 8 / kThreads;   // 16-byte V chunks per thread (2)
constexpr float kRescaleSum = 256.0f;   // a row's block sum above this moves the running max
// Block-sparse history: up to this many kept tiles of a work tile are staged
// in LDS before the key loop (8 bytes each: the tile's (frame, head) plane
// index and its tile index in the frame), so a jump to a kept tile reads no
// memory on the scalar path; later kept tiles take the scalar walk. (The LDS
// ring leaves about 11 KB for it.)
constexpr int kKeptTab = 1280;
constexpr float kFastLimit = 1.8446744e19f;   // 2^64: a block sum above it sends the workgroup to the rescaling loop

// Load tile c: K rows past the valid count and V^T bytes past the plane end
// read as zero through the buffer bounds; V^T columns past the valid count
// inside the plane are finite cache values that meet zero probabilities.
// Thread tid loads the 16-byte chunks tid + 512 i (i = 0, 1) of the K tile
// (byte 16 * chunk) and of the V^T tile (row chunk / 8, column chunk % 8).
// koff = 16 * tid.
__device__ __forceinline__ void load_tile(const TileCursor& c, uint32_t koff, u32x4* kr,
                                          u32x4* vr) {
  const __amdgpu_buffer_rsrc_t rk = tile_k_rsrc<2>(c);
  const __amdgpu_buffer_rsrc_t rv = tile_v_rsrc<2>(c);
  // recompute from koff at every tile rather than keep (or spill) its parts
  uint32_t k = koff;
  asm("" : "+v"(k));
  const uint32_t voff = (k >> 7) * static_cast<uint32_t>(c.vstride * 2) + (k & 0x70u);
#pragma unroll
  for (int i = 0; i < kKChunks; ++i)
    kr[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, i * kThreads * 16, 0));
#pragma unroll
  for (int i = 0; i < kVChunks; ++i)
    vr[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff, i * (kThreads / 8) * c.vstride * 2, 0));
}

__device__ __forceinline__ void store_tile(uint16_t* Ks, uint16_t* Vs, int tid, const u32x4* kr,
                                           const u32x4* vr) {
#pragma unroll
  for (int i = 0; i < kKChunks; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 4, col = c & 15;
    *reinterpret_cast<u32x4*>(&Ks[row * KS + col * 8]) = kr[i];
  }
#pragma unroll
  for (int i = 0; i < kVChunks; ++i) {
    const int c = tid + kThreads * i;
    const int dd = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4*>(&Vs[dd * VS + kc * 8]) = vr[i];
  }
}

// ---- int8 cache (a scale per token and head): tiles are dequantised to bf16
// while staged in registers, so the LDS tiles and everything after them are
// those of the bf16 cache. Thread tid stages the 16 K codes of key row
// tid >> 3 (dims 16 (tid & 7) ..) with that key's scale, and a 4 x 4 block of
// V^T codes (dim rows 4 (tid >> 4) .. +3, keys 4 (tid & 15) .. +3, one
// 4-byte load per row) with those keys' scales: 13 registers in flight, fewer
// than a bf16 tile's 16. Scales of keys past the valid count read as zero.
struct StagedInt8 {
  u32x4 k;
  float ks;
  uint32_t v[4];
  float vs[4];
};

struct StagedBf16 {
  u32x4 k[kKChunks];
  u32x4 v[kVChunks];
};

__device__ __forceinline__ void load_tile_int8(const TileCursor& c, int tid, StagedInt8& st) {
  const __amdgpu_buffer_rsrc_t rk = tile_k_rsrc<kCkInt8>(c);
  const __amdgpu_buffer_rsrc_t rv = tile_v_rsrc<kCkInt8>(c);
  const __amdgpu_buffer_rsrc_t rks = tile_scale_rsrc(c.kst, c);
  const __amdgpu_buffer_rsrc_t rvs = tile_scale_rsrc(c.vst, c);
  const int krow = tid >> 3, kq = tid & 15, dg = tid >> 4;
  st.k = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       rk, static_cast<uint32_t>(tid) * 16u, 0, 0));
  st.ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, krow * 4, 0, 0));
#pragma unroll
  for (int r = 0; r < 4; ++r)
    st.v[r] = __builtin_amdgcn_raw_buffer_load_b32(rv, (4 * dg + r) * c.vstride + 4 * kq, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.vs[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, (4 * kq + i) * 4, 0, 0));
}

// byte b of w as a signed code, times s
__device__ __forceinline__ float dq(uint32_t w, int b, float s) {
  return static_cast<float>(static_cast<int8_t>(w >> (8 * b))) * s;
}

__device__ __forceinline__ void store_tile_int8(uint16_t* Ks, uint16_t* Vs, int tid,
                                                const StagedInt8& st) {
  const int krow = tid >> 3, kc = tid & 7, kq = tid & 15, dg = tid >> 4;
  u32x4 lo, hi;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w = st.k[m];
    const uint32_t a = pack_bf16x2(dq(w, 0, st.ks), dq(w, 1, st.ks));
    const uint32_t b = pack_bf16x2(dq(w, 2, st.ks), dq(w, 3, st.ks));
    if (m < 2) {
      lo[2 * m] = a;
      lo[2 * m + 1] = b;
    } else {
      hi[2 * m - 4] = a;
      hi[2 * m - 3] = b;
    }
  }
  *reinterpret_cast<u32x4*>(&Ks[krow * KS + kc * 16]) = lo;
  *reinterpret_cast<u32x4*>(&Ks[krow * KS + kc * 16 + 8]) = hi;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    u32x2 o;
    o[0] = pack_bf16x2(dq(st.v[r], 0, st.vs[0]), dq(st.v[r], 1, st.vs[1]));
    o[1] = pack_bf16x2(dq(st.v[r], 2, st.vs[2]), dq(st.v[r], 3, st.vs[3]));
    *reinterpret_cast<u32x2*>(&Vs[(4 * dg + r) * VS + 4 * kq]) = o;
  }
}

template <bool kInt8>
using Staged = typename std::conditional<kInt8, StagedInt8, StagedBf16>::type;

template <bool kInt8>
__device__ __forceinline__ void stage_load(const TileCursor& c, uint32_t koff, int tid,
                                           Staged<kInt8>& st) {
  if constexpr (kInt8)
    load_tile_int8(c, tid, st);
  else
    load_tile(c, koff, st.k, st.v);
}

template <bool kInt8>
__device__ __forceinline__ void stage_store(uint16_t* Ks, uint16_t* Vs, int tid,
                                            const Staged<kInt8>& st) {
  if constexpr (kInt8)
    store_tile_int8(Ks, Vs, tid, st);
  else
    store_tile(Ks, Vs, tid, st.k, st.v);
}

// l + lo(a) * lo(b) + hi(a) * hi(b) for packed bf16 pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float l) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b),
                                         l, false);
}

constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // (1.0, 1.0) in bf16

// exp2 of the 16 logits of a block (already relative to the running max),
// packed as two bf16 B operands; returns the sum of the packed values.
__device__ __forceinline__ float block_probs(const f32x16& s, uint32_t ones, bf16x8* p) {
  float l = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    u32x4 pw;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      pw[k] = pack_bf16x2(__builtin_amdgcn_exp2f(s[8 * c + 2 * k]),
                          __builtin_amdgcn_exp2f(s[8 * c + 2 * k + 1]));
      l = dot2_bf16(pw[k], ones, l);
    }
    p[c] = __builtin_bit_cast(bf16x8, pw);
  }
  return l;
}

// Keys of a 32-key block at or beyond `nvalid` (relative to the block) get
// -inf. (Compared as 16 (r / 8) + r % 8 >= nvalid - 8 g: one per-lane value
// against immediates, rather than 16 per-lane key indices the compiler would
// keep in registers across the loop.)
__device__ __forceinline__ void mask_block(f32x16& s, int nvalid, int g) {
  const int lim = nvalid - 8 * g;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (16 * (r >> 3) + (r & 7) >= lim) s[r] = -INFINITY;
}

// Timed text windows on a 32-key block: `word` is the block's visibility
// word for this lane's query row (bit b: key b of the block), and register r
// of lane group g holds key 16 (r / 8) + 8 g + r % 8 (as in mask_block).
__device__ __forceinline__ void window_mask_block(f32x16& s, uint32_t word, int g) {
  const uint32_t wg = word >> (8 * g);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = keep_if_bit(s[r], wg, 16 * (r >> 3) + (r & 7));
}

// Block max of S^T over its 32 keys (both lane halves).
__device__ __forceinline__ float block_max(const f32x16& s) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
  return max_other_half(fmaxf(mx, s[15]));
}

__device__ __forceinline__ bf16x8 lds_op(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// LDS operands of the first two slots of a step, read during the step before.
struct StepOperands {
  bf16x8 v[2];
  bf16x8 k[2];
};

__device__ __forceinline__ const uint16_t* v_operand(const uint16_t* vp, int j) {
  return vp + 16 * (j >> 2) + 32 * (j & 3) * VS;   // keys 16(j/4).., dims 32(j%4)..
}

// One pipeline step. Logits are in log2 units relative to the running max m:
// the queries carry the softmax scale * log2(e), and the QK^T accumulation
// starts from C = -m (negm), so a probability is one exp2 of an accumulator.
// The step issues, slot by slot, PV of the previous block (P^T in p_prev, V^T
// rows at vp) and QK^T of the next block (K rows at kp) on the matrix pipe,
// the LDS reads of the operands two slots ahead (the last two slots read the
// first operands of the next step, at vp_next / kp_next, into `pre`), and the
// exponentials of the current block s_cur with their packing and sum.
// `work` runs in slot 1, once the first MFMAs are queued. Returns the block's
// sum.
template <typename Work>
__device__ __forceinline__ float fused_step(const uint16_t* vp, const uint16_t* kp,
                                            const uint16_t* vp_next, const uint16_t* kp_next,
                                            StepOperands& pre, const bf16x8* p_prev, f32x16* o,
                                            const bf16x8* qf, const f32x16& negm, f32x16& s_next,
                                            const f32x16& s_cur, uint32_t ones, bf16x8* p_cur,
                                            Work&& work) {
  bf16x8 av[8], ak[8];
  av[0] = pre.v[0];
  av[1] = pre.v[1];
  ak[0] = pre.k[0];
  ak[1] = pre.k[1];
  u32x4 pw[2];
  float l0 = 0.f, l1 = 0.f;
  f32x16 s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = i + 2;
    if (j < 8) {
      av[j] = lds_op(v_operand(vp, j));
      ak[j] = lds_op(kp + 16 * j);
    } else {
      pre.v[j - 8] = lds_op(v_operand(vp_next, j - 8));
      pre.k[j - 8] = lds_op(kp_next + 16 * (j - 8));
    }
    const int c = i >> 2, db = i & 3;
    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], p_prev[c], o[db], 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[i], qf[i], i == 0 ? negm : s, 0, 0, 0);
    pw[c][db] = pack_bf16x2(__builtin_amdgcn_exp2f(s_cur[2 * i]),
                            __builtin_amdgcn_exp2f(s_cur[2 * i + 1]));
    if (i & 1)
      l1 = dot2_bf16(pw[c][db], ones, l1);
    else
      l0 = dot2_bf16(pw[c][db], ones, l0);
    // pin this slot's softmax work here: without it instruction selection
    // gathers every exponential of the step after the MFMAs
    asm volatile("" : "+v"(pw[c][db]), "+v"(l0), "+v"(l1));
    if (i == 1) work();
    __builtin_amdgcn_sched_barrier(0);
  }
  s_next = s;
  p_cur[0] = __builtin_bit_cast(bf16x8, pw[0]);
  p_cur[1] = __builtin_bit_cast(bf16x8, pw[1]);
  float l = l0 + l1;
  // materialise the probabilities here, so that they are not sunk past the
  // branch that follows (they must share this block with the MFMAs)
  asm volatile("" : "+v"(p_cur[0]), "+v"(p_cur[1]), "+v"(l));
  return l;
}

// Rare path of a step, taken by the whole wave when some row's block sum
// exceeds kRescaleSum (a probability above it, or many close to it): rows
// whose block max lies above the running max move it there. O (every block
// before this one), the sum before this block, the -m accumulator seed and the
// already issued next block are shifted by the same amount, and the block's
// probabilities are recomputed.
__device__ __forceinline__ float rescale_step(f32x16& negm, float& l_run, f32x16* o,
                                              f32x16& s_cur, f32x16& s_next, uint32_t ones,
                                              bf16x8* p_cur) {
  const float d = fmaxf(block_max(s_cur), 0.f);
  const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] *= alpha;
  l_run *= alpha;
  // whole-vector updates, so that each value keeps its registers across the
  // branch (element-wise updates leave copies on the common path)
  negm = negm - d;
  s_cur = s_cur - d;
  s_next = s_next - d;
  return block_probs(s_cur, ones, p_cur);
}

__device__ __forceinline__ f32x16 qk_block(const uint16_t* kp, const bf16x8* qf) {
  f32x16 s = {};
#pragma unroll
  for (int cd = 0; cd < 8; ++cd)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + 16 * cd),
                                                qf[cd], s, 0, 0, 0);
  return s;
}

template <bool kSparse, bool kInt8>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(const AttnArgs a) {
  constexpr int CK = kInt8 ? kCkInt8 : kCkBf16;   // cache kind of the key-tile walk
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kStages * KT];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kStages * VT];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  // timed-window bits (+ 1 word: block 1 of the last text tile may read one
  // word past the table; its keys are all masked by the valid count)
  __shared__ uint32_t wtab[kWindowWords + 1];
  __shared__ uint2 ktab[kSparse ? kKeptTab : 1];   // kept tiles of the work tile

  const WorkTile wt = map_workgroup(a, BM);
  const AttnItemDev& I = a.items[wt.item];
  const int H = a.heads;
  const int h = wt.head;
  const int q0 = wt.q0;
  const int P = a.rope.P;

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)

  const uint32_t koff_ld = static_cast<uint32_t>(tid) * 16u;
  const TileSeq seq = tile_seq(I, h, q0, BM, P);   // dense, or kept history blocks first
  int kt0, kt1;   // this work tile's logical key tiles
  key_range(a, I, P, wt.part, &kt0, &kt1);
  const int ntiles = kt1 - kt0;
  const int flag_fi = window_flag_segment(I);

  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  stage_window_table(I, wtab, q0, BM, P, tid, kThreads);
  const int PL = plane_tokens(P, CK != kCkBf16);   // token slots of a frame plane
  const uint64_t plane_bytes64 = static_cast<uint64_t>(PL) * kD * elem_bytes<CK>();
  const uint32_t plane_bytes = static_cast<uint32_t>(plane_bytes64);
  int n_tab = 0;   // kept tiles staged (logical tiles kt0 .. kt0 + n_tab - 1)
  if constexpr (kSparse) {
    const int tpf = (P + kKeyTile - 1) / kKeyTile;
    // (a jump multiplies the plane index by a 32-bit plane size)
    n_tab = plane_bytes64 <= 0xFFFFFFFFu ? min(max(0, min(kt1, seq.keep) - kt0), kKeptTab) : 0;
    for (int i = tid; i < n_tab; i += kThreads) {
      const int tile = seq.list[kt0 + i];
      const int fi = tile / tpf;
      const uint32_t pl = static_cast<uint32_t>(I.frames[fi] * H + h);
      ktab[i] = make_uint2(pl, static_cast<uint32_t>(tile - fi * tpf));
    }
  }
  __syncthreads();

  // ---- Q fragments (B operand of S^T = K Q^T): rotated in fp32, times the
  // softmax scale * log2(e), rounded to bf16 ----------------------------------
  const int qrow = q0 + 32 * w + r32;
  const uint32_t* wrow = wtab + window_row_offset(I, q0, qrow, P);   // this row's window bits
  bf16x8 qf[8];
  {
    const float c2 = a.scale_log2;
    bool video;
    int tpos, hpos, wpos;
    query_position(I, a.rope, qrow, &video, &tpos, &hpos, &wpos);
#pragma unroll
    for (int cd = 0; cd < 8; ++cd) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < I.n_q)
        x = *reinterpret_cast<const u32x4*>(I.q + (static_cast<size_t>(qrow) * H + h) * kD +
                                            16 * cd + 8 * g);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float xa = __uint_as_float(x[m] << 16);
        float xb = __uint_as_float(x[m] & 0xFFFF0000u);
        if (video) {
          const int pr = 8 * cd + 4 * g + m;
          const int axis = ax[pr];
          const int pos = axis == 0 ? tpos : (axis == 1 ? hpos : wpos);
          float c, s;
          rope_cos_sin(pos, om[pr], &c, &s);
          const float ya = xa * c - xb * s;
          xb = xa * s + xb * c;
          xa = ya;
        }
        x[m] = pack_bf16x2(xa * c2, xb * c2);
      }
      qf[cd] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int pi_row = (r32 & ~0xC) | ((r32 & 4) << 1) | ((r32 & 8) >> 1);
  const int koff0 = pi_row * KS + 8 * g;          // block 0 K row of this lane
  const int koff1 = (32 + pi_row) * KS + 8 * g;   // block 1
  const int voff = r32 * VS + 8 * g;
  const uint32_t ones = kOnesBf16x2;
  f32x16 o[4];
  f32x16 negm;
  float l_run;
  uint32_t n_resc = 0;   // this wave's rescale steps (diagnostic counters only)
  const char* kbase = static_cast<const char*>(I.k);   // cache bases of the staged kept tiles
  const char* vbase = static_cast<const char*>(I.v);
  const float* kscb = I.k_scale;
  const float* vscb = I.v_scale;

  // The whole key loop, run first without the rescale: the running max stays
  // at block 0's max, and a block sum above kFastLimit only raises a flag
  // (probabilities up to 2^64 stay exact in fp32 and bf16, so nothing before
  // the flag is lost; the flag is raised long before anything could
  // overflow). Without rescale code in the loop the register allocator keeps
  // every block in place. If any row of the workgroup raised the flag, the
  // whole loop runs again, rescaling in place.
  auto attend = [&](auto safe_tag) __attribute__((always_inline)) {
    constexpr bool kSafe = decltype(safe_tag)::value;
    bool over = false;
    // the load cursor runs three tiles ahead of the compute tile; nv0..nv2
    // keep the valid-key counts of the tiles in between
    TileCursor lc;
    // The next tile of the walk: a staged kept tile (its entry read from LDS
    // one step ahead, into ent), else the scalar walk.
    uint2 ent = make_uint2(0u, 0u);
    if constexpr (kSparse) {
      if (n_tab > 3) ent = ktab[3];
    }
    auto advance = [&](int li) __attribute__((always_inline)) {
      if constexpr (kSparse) {
        const int i = li - kt0;   // >= 3: tiles kt0 .. kt0 + 2 are loaded before the loop
        if (i < n_tab) {
          const uint32_t pl = __builtin_amdgcn_readfirstlane(ent.x);
          const uint32_t tix = __builtin_amdgcn_readfirstlane(ent.y);
          if (i + 1 < n_tab) ent = ktab[i + 1];
          const size_t off = static_cast<size_t>(pl) * plane_bytes;
          lc.fi = 0;   // a history frame: never a text segment under timed windows
          lc.p0 = static_cast<int>(tix) * kKeyTile;
          lc.len = P;
          lc.vstride = PL;
          lc.kplane = kbase + off;
          lc.vplane = vbase + off;
          if constexpr (kInt8) {
            lc.kst = kscb + static_cast<size_t>(pl) * PL;
            lc.vst = vscb + static_cast<size_t>(pl) * PL;
          }
          return;
        }
      }
      seq_next<kSparse, CK>(lc, I, h, H, P, seq, li);
    };
    seq_start<kSparse, CK>(lc, I, h, H, P, seq, kt0);
    Staged<kInt8> stg;
    int nv0 = cursor_mask_code(lc, flag_fi);
    stage_load<kInt8>(lc, koff_ld, tid, stg);
    // the last V stage is read once with zero probabilities before it is
    // first written: give it finite contents
    for (int i = tid; i < VT / 8; i += kThreads)
      reinterpret_cast<u32x4*>(Vs + (kStages - 1) * VT)[i] = u32x4{0u, 0u, 0u, 0u};

    // ---- prologue: tiles 0, 1 into LDS stages 0, 1; tile 2 in flight ----------
    stage_store<kInt8>(Ks, Vs, tid, stg);
    int nv1 = 0, nv2 = 0;
    if (ntiles > 1) {
      seq_next<kSparse, CK>(lc, I, h, H, P, seq, kt0 + 1);
      nv1 = cursor_mask_code(lc, flag_fi);
      stage_load<kInt8>(lc, koff_ld, tid, stg);
      stage_store<kInt8>(Ks + KT, Vs + VT, tid, stg);
    }
    if (ntiles > 2) {
      seq_next<kSparse, CK>(lc, I, h, H, P, seq, kt0 + 2);
      nv2 = cursor_mask_code(lc, flag_fi);
      stage_load<kInt8>(lc, koff_ld, tid, stg);
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16{};
    l_run = 0.f;

    // Blocks 2t and 2t+1 are the halves of tile t (stage t % 4). Step 2t still
    // reads V of tile t-1, so tile t+2 goes to stage (t+2) % 4, last read before
    // the barrier that precedes the store.
    // Each tile has two steps, so the two S buffers and the two P buffers swap
    // roles between the steps and the loop carries no register copies.
    // The running max starts at block 0's max (block 0 always has a valid key).
    f32x16 sa = qk_block(Ks + koff0, qf);     // S of block 2t at the top of the loop
    f32x16 sb;                                // S of block 2t+1
    if (nv0 < 32) mask_block(sa, tile_count(nv0), g);
    // (tile 0 is never a text tile under timed windows: the key ranges of such
    // items start on a video tile, so every row sees block 0's valid keys)
    const float m0 = block_max(sa);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      negm[r] = -m0;
      sa[r] -= m0;
    }
    bf16x8 pa[2], pb[2];                      // P of block 2t-1 at the top; of 2t
    pa[0] = pa[1] = bf16x8{};

    // operands of step 0's first slots: V of "tile -1" (the zeroed last stage,
    // met by the zero probabilities pa) and block 1's K rows
    StepOperands pre;
    pre.v[0] = lds_op(v_operand(Vs + (kStages - 1) * VT + voff + 32, 0));
    pre.v[1] = lds_op(v_operand(Vs + (kStages - 1) * VT + voff + 32, 1));
    pre.k[0] = lds_op(Ks + koff1);
    pre.k[1] = lds_op(Ks + koff1 + 16);

#pragma unroll 1
    for (int t = 0; t < ntiles; ++t) {
      const int st = t & (kStages - 1);
      const uint16_t* Kst = Ks + st * KT;
      const uint16_t* Vst = Vs + st * VT;
      const uint16_t* Vprev = Vs + ((t + kStages - 1) & (kStages - 1)) * VT;
      const uint16_t* Knext = Ks + ((t + 1) & (kStages - 1)) * KT;
      const int nvalid = nv0;   // count, sign bit set on a text tile under windows
      int nv3 = 0;
      // Tile t+2: registers -> LDS stage (t+2) % 4, the stage of tile t-2, whose
      // last reads (step 2t-2) completed before this barrier; then start loading
      // tile t+3. Nothing read in this tile's steps lives in that stage, so the
      // barrier needs no fence and the reads already in flight stay in flight.
      auto boundary = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + 2 < ntiles) {
          const int s2 = (t + 2) & (kStages - 1);
          stage_store<kInt8>(Ks + s2 * KT, Vs + s2 * VT, tid, stg);
          if (t + 3 < ntiles) {
            advance(kt0 + t + 3);
            nv3 = cursor_mask_code(lc, flag_fi);
            stage_load<kInt8>(lc, koff_ld, tid, stg);
          }
        }
      };

      // step 2t: PV(2t-1) [pa] + QK(2t+1) [-> sb] | softmax(2t) [sa -> pb]
      if (nvalid < 32) {   // partial tile, or text tile with windows
        if (tile_count(nvalid) < 32) mask_block(sa, tile_count(nvalid), g);
        if (nvalid < 0) window_mask_block(sa, wrow[text_tile_base(I, P, kt0 + t) >> 5], g);
      }
      float lb = fused_step(Vprev + voff + 32, Kst + koff1, Vst + voff, Knext + koff0, pre, pa, o,
                            qf, negm, sb, sa, ones, pb, boundary);
      if constexpr (kSafe) {
        if (__builtin_expect(__any(lb > kRescaleSum), 0)) {
          lb = rescale_step(negm, l_run, o, sa, sb, ones, pb);
          ++n_resc;
        }
      } else {
        over |= lb > kFastLimit;
      }
      l_run += lb;

      // step 2t+1: PV(2t) [pb] + QK(2t+2) [-> sa] | softmax(2t+1) [sb -> pa]
      if (nvalid < BN) {
        if (tile_count(nvalid) < BN) mask_block(sb, tile_count(nvalid) - 32, g);
        if (nvalid < 0) window_mask_block(sb, wrow[(text_tile_base(I, P, kt0 + t) >> 5) + 1], g);
      }
      lb = fused_step(Vst + voff, Knext + koff0, Vst + voff + 32, Knext + koff1, pre, pb, o, qf,
                      negm, sa, sb, ones, pa, [] {});
      if constexpr (kSafe) {
        if (__builtin_expect(__any(lb > kRescaleSum), 0)) {
          lb = rescale_step(negm, l_run, o, sb, sa, ones, pa);
          ++n_resc;
        }
      } else {
        over |= lb > kFastLimit;
      }
      l_run += lb;

      nv0 = nv1;
      nv1 = nv2;
      nv2 = nv3;
    }
    {
      const uint16_t* Vlast = Vs + ((ntiles - 1) & (kStages - 1)) * VT;
      const uint16_t* vp = Vlast + voff + 32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i >> 2, db = i & 3;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(vp + 16 * c + 32 * db * VS), pa[c], o[db], 0, 0, 0);
      }
    }
    return over;
  };
  const bool rerun = __syncthreads_or(attend(std::false_type{}));
  if (rerun) attend(std::true_type{});
  const float m_run = -negm[0];
  if (a.counters != nullptr) add_counts(a.counters, tid, (w == 0 && rerun) ? 1u : 0u, n_resc);

  // The output MFMAs compute across all lanes of the wave: keep them (and
  // everything feeding them) ahead of the per-row store branch below, where
  // lanes past the last query row are switched off.
  asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (wt.part >= 0) {   // split tile: partial result for the merge kernel
    if (qrow < I.n_q)
      store_partial(a, wt.unit, BM, qrow - q0, g, o, 1.0f, m_run, l_tot);
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

int attention_block_m_bf16() { return BM; }

hipError_t launch_attention_bf16(AttnArgs& a, hipStream_t s) {
  const dim3 g(a.grid), b(kThreads);
  if (a.int8 && a.any_sparse)
    hipLaunchKernelGGL((attn_bf16_kernel<true, true>), g, b, 0, s, a);
  else if (a.int8)
    hipLaunchKernelGGL((attn_bf16_kernel<false, true>), g, b, 0, s, a);
  else if (a.any_sparse)
    hipLaunchKernelGGL((attn_bf16_kernel<true, false>), g, b, 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<false, false>), g, b, 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
