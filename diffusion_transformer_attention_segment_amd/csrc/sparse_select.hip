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
//                  workspace [H][n_cand][128]. Reads the history K once.
//   select_kernel  one workgroup per (query block, head): the mean rotated
//                  query (fp32, rows summed in a fixed order), one score per
//                  candidate, then the keep-th largest score by a 4-pass
//                  radix select over order-preserving 32-bit keys, ties to
//                  the lower block index, and the kept indices written in
//                  ascending order through two block scans. Integer counts
//                  only after the scores: the lists are deterministic.
#include "attention_common.h"

namespace segattn {
namespace {

constexpr int kPoolWaves = 4;
constexpr int kSelThreads = 512;
constexpr int kQB = SA_SPARSE_QUERY_BLOCK;   // query rows per block list
constexpr int kChunkRows = 64;               // query rows rotated per LDS pass
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
  const size_t plane = (static_cast<size_t>(frame) * H + h) * static_cast<size_t>(P) * kD;
  float s0 = 0.f, s1 = 0.f;
  if (a.int8) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.item.k) +
                                                             plane) +
                           static_cast<size_t>(r0) * (kD / 2) + lane;
    const float* sc = a.item.k_scale + (static_cast<size_t>(frame) * H + h) * P + r0;
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
  float2 v;
  v.x = s0 * inv;
  v.y = s1 * inv;
  reinterpret_cast<float2*>(a.pooled + (static_cast<size_t>(h) * a.n_cand + c) * kD)[lane] = v;
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

__global__ __launch_bounds__(kSelThreads) void select_kernel(const SelectArgs a) {
  __shared__ float rot[kChunkRows][kD + 4];
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

  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();

  // ---- mean rotated query of the block: 64 rows per pass, 8 threads per row,
  // 8 rotation pairs each; columns summed over rows in row order -------------
  float acc = 0.f;   // column tid (tid < 128)
  for (int c0 = 0; c0 < nrows; c0 += kChunkRows) {
    const int rr = tid >> 3, part = tid & 7;
    const int row = q0 + c0 + rr;
    if (c0 + rr < nrows) {
      bool video;
      int tpos, hpos, wpos;
      query_position(I, a.rope, row, &video, &tpos, &hpos, &wpos);
      const uint16_t* src = I.q + (static_cast<size_t>(row) * H + h) * kD + 16 * part;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(src + 2 * m);
        float xa = __uint_as_float(w << 16), xb = __uint_as_float(w & 0xFFFF0000u);
        if (video) {
          const int pr = 8 * part + m;
          const int axis = ax[pr];
          const int pos = axis == 0 ? tpos : (axis == 1 ? hpos : wpos);
          float cs, sn;
          rope_cos_sin(pos, om[pr], &cs, &sn);
          const float ya = xa * cs - xb * sn;
          xb = xa * sn + xb * cs;
          xa = ya;
        }
        rot[rr][16 * part + 2 * m] = xa;
        rot[rr][16 * part + 2 * m + 1] = xb;
      }
    }
    __syncthreads();
    if (tid < kD) {
      const int n = min(kChunkRows, nrows - c0);
      for (int r = 0; r < n; ++r) acc += rot[r][tid];
    }
    __syncthreads();
  }
  if (tid < kD) pq[tid] = acc / static_cast<float>(nrows);
  __syncthreads();

  // ---- scores of this thread's contiguous run of candidates, as keys that
  // order like the scores (larger score -> larger key) ---------------------------
  const int per = (a.n_cand + kSelThreads - 1) / kSelThreads;
  const int cb = tid * per, ce = min(a.n_cand, cb + per);
  const float* pk = a.pooled + static_cast<size_t>(h) * a.n_cand * kD;
  for (int c = cb; c < ce; ++c) {
    const float4* row = reinterpret_cast<const float4*>(pk + static_cast<size_t>(c) * kD);
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < kD / 4; ++d) {
      const float4 k4 = row[d];
      s = fmaf(pq[4 * d], k4.x, s);
      s = fmaf(pq[4 * d + 1], k4.y, s);
      s = fmaf(pq[4 * d + 2], k4.z, s);
      s = fmaf(pq[4 * d + 3], k4.w, s);
    }
    const uint32_t u = __float_as_uint(s);
    keys[c] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  if (tid == 0) {
    sel_prefix = 0u;
    sel_mask = 0u;
    sel_need = a.keep;
  }
  __syncthreads();

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
    if (tid == 0) {
      const int need = sel_need;
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + static_cast<int>(hist[b]) >= need) break;
        above += static_cast<int>(hist[b]);
      }
      sel_need = need - above;
      sel_prefix = prefix | (static_cast<uint32_t>(b) << shift);
      sel_mask = mask | (255u << shift);
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
