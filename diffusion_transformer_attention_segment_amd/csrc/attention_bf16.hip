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
#include "attention_common.h"

namespace segattn {
namespace {

constexpr int BM = 256;          // query rows per workgroup
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
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before O is rescaled

// Per-thread byte offsets of this thread's 16-byte chunks inside a tile (K) or
// a V^T plane (V, for the two row strides in use).
struct ChunkOffsets {
  uint32_t k[kKChunks];
  uint32_t v_video[kVChunks];
  uint32_t v_text[kVChunks];
};

// Load tile c: K rows past the valid count and V^T bytes past the plane end
// read as zero through the buffer bounds; V^T columns past the valid count
// inside the plane are finite cache values that meet zero probabilities.
__device__ __forceinline__ void load_tile(const TileCursor& c, const ChunkOffsets& off,
                                          bool video, u32x4* kr, u32x4* vr) {
  const __amdgpu_buffer_rsrc_t rk = tile_k_rsrc<2>(c);
  const __amdgpu_buffer_rsrc_t rv = tile_v_rsrc<2>(c);
#pragma unroll
  for (int i = 0; i < kKChunks; ++i)
    kr[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off.k[i], 0, 0));
#pragma unroll
  for (int i = 0; i < kVChunks; ++i)
    vr[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, video ? off.v_video[i] : off.v_text[i],
                                                     0, 0));
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

// exp2(s * c2 - m) for the 16 keys of a block, packed as two bf16 B operands,
// with their fp32 sum folded into l. (The sum uses plain adds: this compiler
// emits v_dot2c_f32_bf16 sequences that read the same source word each time.)
__device__ __forceinline__ void block_probs(const f32x16& s, float c2, float m, float& l,
                                            bf16x8* p) {
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    u32x4 pw;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[8 * c + 2 * k], c2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[8 * c + 2 * k + 1], c2, -m));
      pw[k] = pack_bf16x2(p0, p1);
      l += p0 + p1;
    }
    p[c] = __builtin_bit_cast(bf16x8, pw);
  }
}

// Keys of a 32-key block at or beyond `nvalid` (relative to the block) get -inf.
__device__ __forceinline__ void mask_block(f32x16& s, int nvalid, int g) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 16 * (r >> 3) + 8 * g + (r & 7);
    if (key >= nvalid) s[r] = -INFINITY;
  }
}

// Block max of S^T over its 32 keys (both lane halves), in log2 units.
__device__ __forceinline__ float block_max(const f32x16& s, float c2) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
  return max_other_half(fmaxf(mx, s[15])) * c2;
}

// One pipeline step, one basic block: PV of the previous block (P^T in p_prev,
// V^T rows at vp) and QK^T of the next block (K rows at kp) on the matrix
// pipe, alternating; next to them the max and the exponentials of the current
// block s_cur against the running max m_run. Returns the block max (log2).
__device__ __forceinline__ float fused_step(const uint16_t* vp, const bf16x8* p_prev, f32x16* o,
                                            const uint16_t* kp, const bf16x8* qf, f32x16& s_next,
                                            const f32x16& s_cur, float c2, float m_run,
                                            float& l_run, bf16x8* p_cur) {
  f32x16 s = {};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = i >> 2, db = i & 3;
    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(vp + 16 * c + 32 * db * VS), p_prev[c], o[db], 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + 16 * i),
                                                qf[i], s, 0, 0, 0);
  }
  s_next = s;
  const float mt = block_max(s_cur, c2);
  block_probs(s_cur, c2, m_run, l_run, p_cur);
  // materialise the probabilities here, so that they are not sunk past the
  // branch that follows (they must share this block with the MFMAs)
  asm volatile("" : "+v"(p_cur[0]), "+v"(p_cur[1]), "+v"(l_run));
  return mt;
}

// Rare path of a step: move the running max to the block max where it ran
// ahead by more than the slack, rescale O (which holds every block before this
// one) and the sum accumulated before this block, and recompute the block's
// probabilities against the new max.
__device__ __forceinline__ void rescale_step(float mt, float& m_run, float l_before, float& l_run,
                                             f32x16* o, const f32x16& s_cur, float c2,
                                             bf16x8* p_cur) {
  const bool need = mt > m_run + kRescaleSlack;
  const float mn = need ? mt : m_run;
  const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] *= alpha;
  m_run = mn;
  l_run = l_before * alpha;
  block_probs(s_cur, c2, m_run, l_run, p_cur);
}

__device__ __forceinline__ f32x16 qk_block(const uint16_t* kp, const bf16x8* qf) {
  f32x16 s = {};
#pragma unroll
  for (int cd = 0; cd < 8; ++cd)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + 16 * cd),
                                                qf[cd], s, 0, 0, 0);
  return s;
}

__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kStages * KT];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kStages * VT];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];

  const WorkTile wt = map_workgroup(a, BM);
  const AttnItemDev& I = a.items[wt.item];
  const int H = a.heads;
  const int h = wt.head;
  const int q0 = wt.q0;
  const int P = a.rope.P;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, r32 = lane & 31;

  ChunkOffsets off;
#pragma unroll
  for (int i = 0; i < kKChunks; ++i) {
    const int c = tid + kThreads * i;
    off.k[i] = static_cast<uint32_t>((c >> 4) * kD * 2 + (c & 15) * 16);
  }
#pragma unroll
  for (int i = 0; i < kVChunks; ++i) {
    const int c = tid + kThreads * i;
    off.v_video[i] = static_cast<uint32_t>((c >> 3) * P * 2 + (c & 7) * 16);
    off.v_text[i] = static_cast<uint32_t>((c >> 3) * I.text_cap * 2 + (c & 7) * 16);
  }

  const int tpf = (P + BN - 1) / BN;
  const int ntiles = I.n_frames_kv * tpf + (I.n_text_kv + BN - 1) / BN;

  // the load cursor runs three tiles ahead of the compute tile; nv0..nv2 keep
  // the valid-key counts of the tiles in between
  TileCursor lc;
  lc.fi = 0;
  cursor_enter<2>(lc, I, h, H, P);
  u32x4 kr[kKChunks], vr[kVChunks];
  int nv0 = cursor_nvalid(lc);
  load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);

  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  // the last V stage is read once with zero probabilities before it is first
  // written: give it finite contents
  for (int i = tid; i < VT / 8; i += kThreads)
    reinterpret_cast<u32x4*>(Vs + (kStages - 1) * VT)[i] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- Q fragments (B operand of S^T = K Q^T), rotated in fp32 -------------
  const int qrow = q0 + 32 * w + r32;
  bf16x8 qf[8];
  {
    bool video;
    int tpos, hpos, wpos;
    query_position(I, a.rope, qrow, &video, &tpos, &hpos, &wpos);
#pragma unroll
    for (int cd = 0; cd < 8; ++cd) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qrow < I.n_q)
        x = *reinterpret_cast<const u32x4*>(I.q + (static_cast<size_t>(qrow) * H + h) * kD +
                                            16 * cd + 8 * g);
      if (video) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float xa = __uint_as_float(x[m] << 16);
          const float xb = __uint_as_float(x[m] & 0xFFFF0000u);
          const int pr = 8 * cd + 4 * g + m;
          const int axis = ax[pr];
          const int pos = axis == 0 ? tpos : (axis == 1 ? hpos : wpos);
          float c, s;
          rope_cos_sin(pos, om[pr], &c, &s);
          x[m] = pack_bf16x2(xa * c - xb * s, xa * s + xb * c);
        }
      }
      qf[cd] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // ---- prologue: tiles 0, 1 into LDS stages 0, 1; tile 2 in flight ----------
  store_tile(Ks, Vs, tid, kr, vr);
  int nv1 = 0, nv2 = 0;
  if (ntiles > 1) {
    cursor_next<2>(lc, I, h, H, P);
    nv1 = cursor_nvalid(lc);
    load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
    store_tile(Ks + KT, Vs + VT, tid, kr, vr);
  }
  if (ntiles > 2) {
    cursor_next<2>(lc, I, h, H, P);
    nv2 = cursor_nvalid(lc);
    load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
  }
  __syncthreads();

  const int pi_row = (r32 & ~0xC) | ((r32 & 4) << 1) | ((r32 & 8) >> 1);
  const int koff0 = pi_row * KS + 8 * g;          // block 0 K row of this lane
  const int koff1 = (32 + pi_row) * KS + 8 * g;   // block 1
  const int voff = r32 * VS + 8 * g;
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  // Blocks 2t and 2t+1 are the halves of tile t (stage t % 4). Step 2t still
  // reads V of tile t-1, so tile t+2 goes to stage (t+2) % 4, last read before
  // the barrier that precedes the store.
  // Each tile has two steps, so the two S buffers and the two P buffers swap
  // roles between the steps and the loop carries no register copies.
  f32x16 sa = qk_block(Ks + koff0, qf);     // S of block 2t at the top of the loop
  f32x16 sb;                                // S of block 2t+1
  if (nv0 < 32) mask_block(sa, nv0, g);
  float m_run = block_max(sa, c2);          // block 0 always has a valid key
  bf16x8 pa[2], pb[2];                      // P of block 2t-1 at the top; of 2t
  pa[0] = pa[1] = bf16x8{};

#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & (kStages - 1);
    const uint16_t* Kst = Ks + st * KT;
    const uint16_t* Vst = Vs + st * VT;
    const uint16_t* Vprev = Vs + ((t + kStages - 1) & (kStages - 1)) * VT;
    const uint16_t* Knext = Ks + ((t + 1) & (kStages - 1)) * KT;
    const int nvalid = nv0;
    __syncthreads();
    // tile t+2: registers -> LDS stage (t+2) % 4; start loading tile t+3
    int nv3 = 0;
    if (t + 2 < ntiles) {
      const int s2 = (t + 2) & (kStages - 1);
      store_tile(Ks + s2 * KT, Vs + s2 * VT, tid, kr, vr);
      if (t + 3 < ntiles) {
        cursor_next<2>(lc, I, h, H, P);
        nv3 = cursor_nvalid(lc);
        load_tile(lc, off, lc.fi < I.n_frames_kv, kr, vr);
      }
    }

    // step 2t: PV(2t-1) [pa] + QK(2t+1) [-> sb] | softmax(2t) [sa -> pb]
    if (nvalid < 32) mask_block(sa, nvalid, g);
    float l_before = l_run;
    float mt = fused_step(Vprev + voff + 32, pa, o, Kst + koff1, qf, sb, sa, c2, m_run, l_run, pb);
    if (__any(mt > m_run + kRescaleSlack))
      rescale_step(mt, m_run, l_before, l_run, o, sa, c2, pb);

    // step 2t+1: PV(2t) [pb] + QK(2t+2) [-> sa] | softmax(2t+1) [sb -> pa]
    if (nvalid < BN) mask_block(sb, nvalid - 32, g);
    l_before = l_run;
    mt = fused_step(Vst + voff, pb, o, Knext + koff0, qf, sa, sb, c2, m_run, l_run, pa);
    if (__any(mt > m_run + kRescaleSlack))
      rescale_step(mt, m_run, l_before, l_run, o, sb, c2, pa);

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

  // The output MFMAs compute across all lanes of the wave: keep them (and
  // everything feeding them) ahead of the per-row store branch below, where
  // lanes past the last query row are switched off.
  asm volatile("" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));

  // ---- epilogue ----------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
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
  hipLaunchKernelGGL(attn_bf16_kernel, dim3(a.total_tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
