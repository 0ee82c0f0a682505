// segment_attention, bf16 cache: fused Q-RoPE + flash-style attention over a
// gathered key set (kept history frames via an index list, the current
// segment's frames, the text slot), bf16 MFMA on gfx950, fp32 accumulation.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// sections "How one segment is made" (joint attention of the segment's video
// and text tokens, 16 heads of 128, 3D RoPE, reading history from a KV cache)
// and "The 4090 preset" (a picked subset of past frames is attended).
//
// Work decomposition. One workgroup = 4 waves = 128 query rows of one head of
// one session; each wave owns 32 rows. Key tiles of 64 keys never straddle a
// frame (a frame of P tokens is ceil(P/64) tiles), so a tile's address is one
// frame-plane base plus a row offset and the frame list is read once per tile.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, 32x32 output, K = 16):
//   S^T = K . Q^T   A = K rows (keys), B = Q^T (queries = lanes % 32)
//   O^T = V^T . P^T A = V^T rows (dims), B = P^T (queries = lanes % 32)
// The S^T accumulator of lane l holds, for query l % 32, keys
//   8*(r/4) + 4*(l/32) + r%4 of the A rows (register r). Loading K row
//   pi(r) = r with bits 2 and 3 swapped into A row r makes lane-group g hold the
//   contiguous keys 16c + 8g .. 16c + 8g + 7 in registers 8c .. 8c + 7, which
//   is exactly the B-operand layout P^T needs -- so P never leaves registers,
//   and V^T (stored transposed in the cache) is read as contiguous 16 bytes.
#include "device_common.h"

namespace segattn {
namespace {

constexpr int BM = 128;          // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int kThreads = 256;
constexpr int KS = kD + 8;       // LDS row stride of the K tile (elements)
constexpr int VS = BN + 8;       // LDS row stride of the V^T tile (elements)
constexpr float kRescaleSlack = 8.0f;   // log2 headroom before O is rescaled

struct TileDesc {
  const uint16_t* kb;   // K row 0 of the tile
  const uint16_t* vb;   // V^T column 0 of the tile (row stride vstride)
  int vstride;
  int nvalid;           // valid keys in the tile (1..64)
};

__device__ __forceinline__ TileDesc tile_at(const AttnItemDev& I, int t, int tpf, int nvid,
                                            int h, int H, int P) {
  TileDesc d;
  if (t < nvid) {
    const int fi = t / tpf;
    const int p0 = (t - fi * tpf) * BN;
    const int frame = I.frames[fi];
    const size_t plane = (static_cast<size_t>(frame) * H + h) * static_cast<size_t>(P) * kD;
    d.kb = static_cast<const uint16_t*>(I.k) + plane + static_cast<size_t>(p0) * kD;
    d.vb = static_cast<const uint16_t*>(I.v) + plane + p0;
    d.vstride = P;
    d.nvalid = min(BN, P - p0);
  } else {
    const int p0 = (t - nvid) * BN;
    const size_t plane = static_cast<size_t>(h) * I.text_cap * kD;
    d.kb = static_cast<const uint16_t*>(I.k_text) + plane + static_cast<size_t>(p0) * kD;
    d.vb = static_cast<const uint16_t*>(I.v_text) + plane + p0;
    d.vstride = I.text_cap;
    d.nvalid = min(BN, I.n_text_kv - p0);
  }
  return d;
}

__device__ __forceinline__ void load_tile(const TileDesc& d, int tid, u32x4* kr, u32x4* vr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 4, col = c & 15;
    kr[i] = row < d.nvalid
                ? *reinterpret_cast<const u32x4*>(d.kb + static_cast<size_t>(row) * kD + col * 8)
                : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int dd = c >> 3, kc = c & 7;
    vr[i] = 8 * kc < d.nvalid
                ? *reinterpret_cast<const u32x4*>(d.vb + static_cast<size_t>(dd) * d.vstride + kc * 8)
                : u32x4{0u, 0u, 0u, 0u};
  }
}

__device__ __forceinline__ void store_tile(uint16_t* Ks, uint16_t* Vs, int tid, const u32x4* kr,
                                           const u32x4* vr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 4, col = c & 15;
    *reinterpret_cast<u32x4*>(&Ks[row * KS + col * 8]) = kr[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int dd = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4*>(&Vs[dd * VS + kc * 8]) = vr[i];
  }
}

__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(const AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kD * VS];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];

  // XCD-aware order: workgroups go round-robin over the 8 XCDs, so give each
  // XCD a contiguous run of logical tiles (same head => shared K/V in its L2).
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b & 7, idx = b >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = xcd * per + min(xcd, rem) + idx;

  int it = 0;
#pragma unroll 1
  for (int j = 1; j < a.n_items; ++j)
    if (logical >= a.items[j].tile_begin) it = j;
  const AttnItemDev& I = a.items[it];
  const int local = logical - I.tile_begin;
  const int H = a.heads;
  const int h = local / I.q_tiles;
  const int q0 = (local - h * I.q_tiles) * BM;
  const int P = a.rope.P;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, r32 = lane & 31;

  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();

  // ---- Q fragments (B operand of S^T = K Q^T), rotated in fp32 -------------
  const int qrow = q0 + 32 * w + r32;
  bf16x8 qf[8];
  {
    int tpos = 0, hpos = 0, wpos = 0;
    const bool video = qrow < I.n_q_video;
    if (video) {
      const int f = qrow / P, p = qrow - (qrow / P) * P;
      tpos = I.frame0_q + f;
      hpos = p / a.rope.lat_w;
      wpos = p - hpos * a.rope.lat_w;
    }
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

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  const int tpf = (P + BN - 1) / BN;
  const int nvid = I.n_frames_kv * tpf;
  const int ntiles = nvid + (I.n_text_kv + BN - 1) / BN;

  // K row this lane feeds into A row r32 (bits 2 and 3 swapped)
  const int pi_row = (r32 & ~0xC) | ((r32 & 4) << 1) | ((r32 & 8) >> 1);

  u32x4 kr[4], vr[4];
  TileDesc cur = tile_at(I, 0, tpf, nvid, h, H, P);
  load_tile(cur, tid, kr, vr);

#pragma unroll 1
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile(Ks, Vs, tid, kr, vr);
    __syncthreads();
    const int nvalid = cur.nvalid;
    if (t + 1 < ntiles) {
      cur = tile_at(I, t + 1, tpf, nvid, h, H, P);
      load_tile(cur, tid, kr, vr);
    }

    // ---- S^T = K Q^T for two 32-key blocks --------------------------------
    f32x16 s[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      s[bk] = f32x16{};
      const uint16_t* krow = &Ks[(32 * bk + pi_row) * KS + 8 * g];
#pragma unroll
      for (int cd = 0; cd < 8; ++cd) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(krow + 16 * cd);
        s[bk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[cd], s[bk], 0, 0, 0);
      }
    }
    if (nvalid < BN) {
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * bk + 16 * (r >> 3) + 8 * g + (r & 7);
          if (key >= nvalid) s[bk][r] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain, lazy rescale) ------------------------
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c2;
    const bool need = mt > m_run + kRescaleSlack;
    if (__any(need)) {
      const float mn = need ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    float lsum = 0.f;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[bk][r], c2, -m_run));
        s[bk][r] = p;
        lsum += p;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int bk = cc >> 1, hh = (cc & 1) * 8;
      u32x4 pw;
#pragma unroll
      for (int m = 0; m < 4; ++m) pw[m] = pack_bf16x2(s[bk][hh + 2 * m], s[bk][hh + 2 * m + 1]);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 av =
            *reinterpret_cast<const bf16x8*>(&Vs[(32 * db + r32) * VS + 16 * cc + 8 * g]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf, o[db], 0, 0, 0);
      }
    }
  }

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
