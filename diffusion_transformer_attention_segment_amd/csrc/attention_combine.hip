// Merge of split attention tiles: each query tile of the last partial round
// was computed as split_k parts over disjoint key ranges; part k left, per
// row, its running max m_k (log2 units), the sum l_k of the exponentials
// against it and the unnormalised output O_k. The merged row is
//   m = max_k m_k,  w_k = 2^(m_k - m),  out = (sum_k w_k O_k) / (sum_k w_k l_k),
//   lse = (m + log2 sum_k w_k l_k) * ln 2,
// combined in part order (deterministic). This is the exact softmax over the
// union of the key ranges: softmax over a key set split in two equals the
// max/sum-reweighted merge of the two partial softmaxes.
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache", section
// "How one segment is made" (one joint attention over cached and own keys).
#include "attention_common.h"

namespace segattn {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kRowsPerBlock = kCombineThreads / 4;   // four threads per row, 32 dims each

// grid: (split tiles) x (block_m / 64); thread (row, quarter) of the tile
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const AttnArgs a, int block_m) {
  const int logical = a.n_full + blockIdx.x;
  int it = 0;
  for (int j = 1; j < a.n_items; ++j)
    if (logical >= a.items[j].tile_begin) it = j;
  const AttnItemDev& I = a.items[it];
  const int local = logical - I.tile_begin;
  const int h = local / I.q_tiles;
  const int q0 = (local - h * I.q_tiles) * block_m;
  const int row = blockIdx.y * kRowsPerBlock + (threadIdx.x >> 2);
  const int quarter = threadIdx.x & 3;
  const int qrow = q0 + row;
  if (row >= block_m || qrow >= I.n_q) return;
  const int K = a.split_k;
  const size_t unit_floats = static_cast<size_t>(block_m) * kPartialStride;
  const size_t m_off = static_cast<size_t>(block_m) * kD + row;
  const size_t l_off = static_cast<size_t>(block_m) * (kD + 1) + row;
  const float* base = a.ws + static_cast<size_t>(blockIdx.x) * K * unit_floats;

  float m = -INFINITY;
  for (int k = 0; k < K; ++k) m = fmaxf(m, base[k * unit_floats + m_off]);
  float acc[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.f;
  float l = 0.f;
  for (int k = 0; k < K; ++k) {
    const float* u = base + k * unit_floats;
    const float wk = __builtin_amdgcn_exp2f(u[m_off] - m);
    l += wk * u[l_off];
    const float4* src = reinterpret_cast<const float4*>(u + static_cast<size_t>(row) * kD + 32 * quarter);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 v = src[c];
      acc[4 * c] += wk * v.x;
      acc[4 * c + 1] += wk * v.y;
      acc[4 * c + 2] += wk * v.z;
      acc[4 * c + 3] += wk * v.w;
    }
  }
  const float inv = 1.0f / l;
  uint16_t* out = I.out + (static_cast<size_t>(qrow) * a.heads + h) * kD + 32 * quarter;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[8 * c + 2 * e] * inv, acc[8 * c + 2 * e + 1] * inv);
    *reinterpret_cast<u32x4*>(out + 8 * c) = w;
  }
  if (I.lse != nullptr && quarter == 0)
    I.lse[static_cast<size_t>(qrow) * a.heads + h] = (m + __log2f(l)) * 0.6931471805599453f;
}

}  // namespace

hipError_t launch_attention_combine(const AttnArgs& a, int block_m, hipStream_t s) {
  const int n = a.total_tiles - a.n_full;
  if (n <= 0) return hipSuccess;
  const int row_blocks = (block_m + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(combine_kernel, dim3(n, row_blocks), dim3(kCombineThreads), 0, s, a, block_m);
  return hipGetLastError();
}

}  // namespace segattn
