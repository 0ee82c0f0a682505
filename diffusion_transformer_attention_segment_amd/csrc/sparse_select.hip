// sparse_select: block lists for block-sparse history attention.
//
// Source: "Hy-Nomas en una RTX 4090" (inferencekey.com), section "El preset
// de una GPU": after the first denoising steps the preset's sparse attention
// keeps a quarter of the candidate video blocks. The block size, the query
// block and the pooled score are readings: candidate blocks are the 64-token
// key tiles of the history frames, a query block is 256 rows, and the score is
// the mean rotated query of the block dotted with the mean stored key of the
// candidate.
//
// Two kernels:
//   pool_k_kernel  one wave per candidate block: the mean of its <= 64 stored
//                  keys (e4m3 codes times the plane scale, int8 codes times
//                  their token's scale), fp32, into the
//                  workspace [H][128][n_cand] (dim-major). Reads the history K once.
//   select_kernel  one workgroup per (query block, head): the mean rotated
//                  query (fp32, rows summed in a fixed order), one score per
//                  candidate, then the keep-th largest score by a 4-pass
//                  radix select over order-preserving 32-bit keys, ties to
//                  the lower block index, and the kept indices written in
//                  ascending order through two block scans. Integer counts
//                  only after the scores: the lists are deterministic.
#include <mutex>

#include "attention_common.h"

// Pooled keys of sa_sparse_select_noalloc: [H][128][n_cand] fp32 in the
// library's own device memory, one copy per GPU. Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) float scratch[SA_SPARSE_SCRATCH_BYTES / sizeof(float)];

namespace segattn {
namespace {

constexpr int kPoolWaves = 4;
constexpr int kSelThreads = 512;
constexpr int kQB = SA_SPARSE_QUERY_BLOCK;   // query rows per block list
constexpr int kRowGroups = kSelThreads / 8;  // query rows rotated at a time (8 threads each)
constexpr int kSelLut = 2048;                // cos/sin entries of a query block's table
constexpr int kPerThread = (kMaxCandidates + kSelThreads - 1) / kSelThreads;   // 16

__global__ __launch_bounds__(64 * kPoolWaves) void pool_k_kernel(const SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * kPoolWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.y;
  if (c >= a.n_cand) return;
  const int P = a.rope.P, H = a.heads;
  const int tpf = (P + kKeyTile - 1) / kKeyTile;
  const int fi = c / tpf, j = c - fi * tpf;
  const int frame = a.item.frames[fi];
  const int r0 = j * kKeyTile, n = min(kKeyTile, P - r0);
  const int PL = plane_tokens(P, a.int8 || a.fp8);   // token slots of a plane
  const size_t plane = (static_cast<size_t>(frame) * H + h) * static_cast<size_t>(PL) * kD;
  float s0 = 0.f, s1 = 0.f;
  if (a.int8) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.item.k) +
                                                             plane) +
                           static_cast<size_t>(r0) * (kD / 2) + lane;
    const float* sc = a.item.k_scale + (static_cast<size_t>(frame) * H + h) * PL + r0;
#pragma unroll 8
    for (int r = 0; r < n; ++r) {
      const uint32_t w = base[static_cast<size_t>(r) * (kD / 2)];
      const float scl = sc[r];
      s0 += static_cast<float>(static_cast<int8_t>(w)) * scl;
      s1 += static_cast<float>(static_cast<int8_t>(w >> 8)) * scl;
    }
  } else if (!a.fp8) {
    const uint32_t* base =
        reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.item.k) + plane) +
        static_cast<size_t>(r0) * (kD / 2) + lane;
#pragma unroll 8
    for (int r = 0; r < n; ++r) {
      const uint32_t w = base[static_cast<size_t>(r) * (kD / 2)];
      s0 += __uint_as_float(w << 16);
      s1 += __uint_as_float(w & 0xFFFF0000u);
    }
  } else {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.item.k) +
                                                             plane) +
                           static_cast<size_t>(r0) * (kD / 2) + lane;
#pragma unroll 8
    for (int r = 0; r < n; ++r) {
      typedef float f32x2v __attribute__((ext_vector_type(2)));
      const f32x2v f = __builtin_amdgcn_cvt_pk_f32_fp8(
          static_cast<int>(base[static_cast<size_t>(r) * (kD / 2)]), false);
      s0 += f[0];
      s1 += f[1];
    }
    const float sc = a.item.k_scale[static_cast<size_t>(frame) * H + h];
    s0 *= sc;
    s1 *= sc;
  }
  const float inv = 1.0f / static_cast<float>(n);
  // dim-major [H][128][n_cand]: the scores read one dim of consecutive
  // candidates per load
  float* dst = a.pooled + (static_cast<size_t>(h) * kD + 2 * lane) * a.n_cand + c;
  dst[0] = s0 * inv;
  dst[a.n_cand] = s1 * inv;
}

// Exclusive prefix sum of v over the workgroup's threads (in thread order);
// *total gets the sum. tmp: kSelThreads / 64 ints of LDS.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    const int t = tmp[i];
    before += i < w ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// The rotation table of a query block: the t band of the frames its video
// rows span (f_lo ..), the h band of every latent row and the w band of every
// column, each entry from the same fp64-reduced angle as rope_cos_sin, so a
// lookup and the direct evaluation agree bit for bit.
struct QueryLut {
  int nt, nh, nw;   // pairs per band
  int f_lo, nf;     // first frame (within the segment) and frame count
  int lat_h;
  int size;         // entries: nf * nt + lat_h * nh + lat_w * nw
};

__device__ __forceinline__ QueryLut query_lut_shape(const AttnItemDev& I, const RopeParams& r,
                                                    int q0, int nrows) {
  QueryLut s;
  s.nt = r.split0 / 2;
  s.nh = r.split1 / 2;
  s.nw = r.split2 / 2;
  s.lat_h = r.P / r.lat_w;
  const int v_end = min(q0 + nrows, I.n_q_video);
  s.f_lo = q0 / r.P;
  s.nf = v_end > q0 ? (v_end - 1) / r.P - s.f_lo + 1 : 0;
  s.size = s.nf * s.nt + s.lat_h * s.nh + r.lat_w * s.nw;
  return s;
}

__device__ void build_query_lut(float2* lut, const QueryLut& s, const AttnItemDev& I,
                                const RopeParams& r) {
  for (int i = threadIdx.x; i < s.size; i += kSelThreads) {
    int pair, pos;
    if (i < s.nf * s.nt) {
      const int f = i / s.nt;
      pair = i - f * s.nt;
      pos = I.frame0_q + s.f_lo + f;
    } else if (i < s.nf * s.nt + s.lat_h * s.nh) {
      const int j = i - s.nf * s.nt;
      pos = j / s.nh;
      pair = s.nt + (j - pos * s.nh);
    } else {
      const int j = i - s.nf * s.nt - s.lat_h * s.nh;
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

__device__ __forceinline__ float2 query_lut_get(const float2* lut, const QueryLut& s, int pair,
                                                int f, int hh, int ww) {
  if (pair < s.nt) return lut[(f - s.f_lo) * s.nt + pair];
  if (pair < s.nt + s.nh) return lut[s.nf * s.nt + hh * s.nh + (pair - s.nt)];
  return lut[s.nf * s.nt + s.lat_h * s.nh + ww * s.nw + (pair - s.nt - s.nh)];
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectArgs a) {
  __shared__ float2 lut[kSelLut];
  __shared__ float wsum[kSelThreads / 64][kD];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  __shared__ float pq[kD];
  __shared__ uint32_t keys[kMaxCandidates];
  __shared__ uint32_t hist[256];
  __shared__ int scan_tmp[kSelThreads / 64];
  __shared__ uint32_t sel_prefix, sel_mask;
  __shared__ int sel_need;

  const AttnItemDev& I = a.item;
  const int tid = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, H = a.heads;
  const int q0 = qt * kQB;
  const int nrows = min(kQB, I.n_q - q0);

  const QueryLut ls = query_lut_shape(I, a.rope, q0, nrows);
  const bool use_lut = ls.size <= kSelLut;
  if (use_lut) {
    build_query_lut(lut, ls, I, a.rope);
  } else if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();

  // ---- mean rotated query of the block: 8 threads per row, 8 rotation pairs
  // (16 dims) each; every thread sums its dims over its rows (rr, rr + 64, ...)
  // in registers, then the 64 row groups are reduced in a fixed order (lanes,
  // then waves), so the mean is deterministic -------------------------------------
  const int rr = tid >> 3, part = tid & 7;
  float ps[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) ps[i] = 0.f;
  for (int c0 = 0; c0 < nrows; c0 += kRowGroups) {
    if (c0 + rr < nrows) {
      const int row = q0 + c0 + rr;
      bool video;
      int tpos, hpos, wpos;
      query_position(I, a.rope, row, &video, &tpos, &hpos, &wpos);
      const uint16_t* src = I.q + (static_cast<size_t>(row) * H + h) * kD + 16 * part;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 8);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t wd = m < 4 ? w0[m] : w1[m - 4];
        float xa = __uint_as_float(wd << 16), xb = __uint_as_float(wd & 0xFFFF0000u);
        if (video) {
          const int pr = 8 * part + m;
          float cs, sn;
          if (use_lut) {
            const float2 e = query_lut_get(lut, ls, pr, tpos - I.frame0_q, hpos, wpos);
            cs = e.x;
            sn = e.y;
          } else {
            const int axis = ax[pr];
            rope_cos_sin(axis == 0 ? tpos : (axis == 1 ? hpos : wpos), om[pr], &cs, &sn);
          }
          const float ya = xa * cs - xb * sn;
          xb = xa * sn + xb * cs;
          xa = ya;
        }
        ps[2 * m] += xa;
        ps[2 * m + 1] += xb;
      }
    }
  }
  // lanes of one wave with the same dims differ in lane bits 3-5 (rows)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ps[i] += __shfl_xor(ps[i], 8);
    ps[i] += __shfl_xor(ps[i], 16);
    ps[i] += __shfl_xor(ps[i], 32);
  }
  if ((tid & 63) < 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) wsum[tid >> 6][16 * part + i] = ps[i];
  }
  __syncthreads();
  float acc = 0.f;   // column tid (tid < 128), waves in order
  if (tid < kD) {
#pragma unroll
    for (int i = 0; i < kSelThreads / 64; ++i) acc += wsum[i][tid];
  }
  if (tid < kD) pq[tid] = acc / static_cast<float>(nrows);
  __syncthreads();

  // ---- one score per candidate (candidates tid, tid + 512, ...: a load reads
  // one dim of 64 consecutive candidates), as a key that orders like the score
  // (larger score -> larger key); dims in order, so the score is the same
  // fp32 chain whatever the layout ----------------------------------------------
  const float* pk = a.pooled + static_cast<size_t>(h) * kD * a.n_cand;
  for (int c = tid; c < a.n_cand; c += kSelThreads) {
    float s = 0.f;
#pragma unroll 16
    for (int d = 0; d < kD; ++d) s = fmaf(pq[d], pk[static_cast<size_t>(d) * a.n_cand + c], s);
    const uint32_t u = __float_as_uint(s);
    keys[c] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  if (tid == 0) {
    sel_prefix = 0u;
    sel_mask = 0u;
    sel_need = a.keep;
  }
  __syncthreads();
  // from here on each thread owns a contiguous run of candidates (index order)
  const int per = (a.n_cand + kSelThreads - 1) / kSelThreads;
  const int cb = tid * per, ce = min(a.n_cand, cb + per);

  // ---- radix select of the keep-th largest key, 8 bits per pass from the top --
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t prefix = sel_prefix, mask = sel_mask;
    for (int c = cb; c < ce; ++c) {
      const uint32_t k = keys[c];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // the highest bin b whose keys from b up reach `need`: lane l holds bins
      // 255 - 4 l .. 252 - 4 l; counts of the bins above come from a scan
      // over the lanes, and the first lane that reaches `need` decides
      const int need = sel_need;
      int c[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = static_cast<int>(hist[255 - 4 * tid - i]);
        s += c[i];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (tid >= o) incl += y;
      }
      const unsigned long long hit = __ballot(incl >= need);
      if (tid == __ffsll(static_cast<long long>(hit)) - 1) {
        int above = incl - s, b = 255 - 4 * tid;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          if (above + c[i] >= need) break;
          above += c[i];
          --b;
        }
        sel_need = need - above;
        sel_prefix = prefix | (static_cast<uint32_t>(b) << shift);
        sel_mask = mask | (255u << shift);
      }
    }
    __syncthreads();
  }
  // threshold key T: every key above it is kept, and the first sel_need keys
  // equal to it in index order
  const uint32_t T = sel_prefix;
  const int need_eq = sel_need;
  int n_eq = 0;
  for (int c = cb; c < ce; ++c) n_eq += keys[c] == T;
  int total;
  int eq_before = block_exclusive_scan(n_eq, scan_tmp, &total);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int c = cb; c < ce; ++c) {
      const uint32_t k = keys[c];
      const bool eq = k == T;
      n_sel += (k > T) || (eq && e < need_eq);
      e += eq;
    }
  }
  int pos = block_exclusive_scan(n_sel, scan_tmp, &total);
  int32_t* out = a.out + (static_cast<size_t>(h) * I.q_tiles + qt) * a.keep;
  {
    int e = eq_before;
    for (int c = cb; c < ce; ++c) {
      const uint32_t k = keys[c];
      const bool eq = k == T;
      if (((k > T) || (eq && e < need_eq)) && pos < a.keep) out[pos++] = c;
      e += eq;
    }
  }
}

}  // namespace

hipError_t sparse_select_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_sparse_select(const SelectArgs& a, hipStream_t s) {
  static_assert(kPerThread <= 16, "a thread's candidate run stays short");
  hipLaunchKernelGGL(pool_k_kernel, dim3((a.n_cand + kPoolWaves - 1) / kPoolWaves, a.heads),
                     dim3(64 * kPoolWaves), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(a.item.q_tiles, a.heads), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
