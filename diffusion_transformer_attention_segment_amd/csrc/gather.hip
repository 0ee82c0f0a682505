// history_gather (materialising frame gather) and kv_dequant (e4m3 or int8
// -> bf16).
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// section "The 4090 preset": before each segment the picked past frames are
// restored from the archive to the GPU; "Hy-Nomas en una RTX 4090",
// section "El preset de una GPU": the cache is stored in a narrow format and
// computed in BF16.
//
// Both kernels are HBM-bound copies: gather moves 2 * plane_bytes per frame in
// and out; dequant reads 1 byte and writes 2 bytes per element. The gather's
// loads and stores are non-temporal (every byte is touched once; about 10 %
// faster). The dequant's are not: there the same hint cost 30 %.
#include "device_common.h"

namespace segattn {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kChunksPerThread = 4;   // 16-byte chunks in flight per thread

// grid: (chunks of a frame's plane / (256 * 4), n frames, 2 planes (K, V))
__global__ __launch_bounds__(kGatherThreads) void gather_kernel(const GatherArgs a) {
  const int i = blockIdx.y;
  const int which = blockIdx.z;
  const int frame = a.frames[i];
  const char* src = static_cast<const char*>(which ? a.src_v : a.src_k) + frame * a.plane_bytes;
  char* dst = static_cast<char*>(which ? a.dst_v : a.dst_k) + static_cast<int64_t>(i) * a.plane_bytes;
  const int64_t n16 = a.plane_bytes >> 4;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kGatherThreads * kChunksPerThread;
  u32x4 x[kChunksPerThread];
#pragma unroll
  for (int j = 0; j < kChunksPerThread; ++j) {
    const int64_t c = base + threadIdx.x + j * kGatherThreads;
    if (c < n16) x[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + c);
  }
#pragma unroll
  for (int j = 0; j < kChunksPerThread; ++j) {
    const int64_t c = base + threadIdx.x + j * kGatherThreads;
    if (c < n16) __builtin_nontemporal_store(x[j], reinterpret_cast<u32x4*>(dst) + c);
  }
  // the frame's scales (fp8: one per head; int8: one per token and head),
  // spread over the frame's blocks
  if (a.src_ks != nullptr) {
    const float* ss = (which ? a.src_vs : a.src_ks) + static_cast<int64_t>(frame) * a.scale_floats;
    float* ds = (which ? a.dst_vs : a.dst_ks) + static_cast<int64_t>(i) * a.scale_floats;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * kGatherThreads + threadIdx.x;
         e < a.scale_floats; e += static_cast<int64_t>(gridDim.x) * kGatherThreads)
      ds[e] = ss[e];
  }
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xFu;
  const uint32_t m = c & 0x7u;
  float v;
  if (e == 0) {
    v = static_cast<float>(m) * 0.001953125f;          // m * 2^-9
  } else if (e == 15 && m == 7) {
    v = __uint_as_float(0x7FC00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  }
  return __uint_as_float(__float_as_uint(v) | sign);
}

// grid: (ceil(chunks / 256), n planes (frames or 1), H * 2), 8-byte chunks.
// Each thread converts 8 consecutive bytes of one (frame, head) plane into
// 16 bytes of bf16, so that a wave's stores are one contiguous run.
constexpr int kDqChunk = 8;
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs a) {
  const int i = blockIdx.y;
  const int h = blockIdx.z >> 1;
  const int which = blockIdx.z & 1;        // 0: K [tok][128], 1: V^T [128][tok]
  const int frame = a.frames != nullptr ? a.frames[i] : 0;
  const float scale = (which ? a.src_vs : a.src_ks)[static_cast<int64_t>(frame) * a.heads + h];
  const uint8_t* src = (which ? a.src_v : a.src_k) +
                       (static_cast<int64_t>(frame) * a.heads + h) * a.src_len * kD;
  uint16_t* dst = (which ? a.dst_v : a.dst_k) +
                  (static_cast<int64_t>(i) * a.heads + h) * a.dst_len * kD;
  const int c = blockIdx.x * 256 + threadIdx.x;   // chunk index
  int row, col, src_row_len, dst_row_len, row_valid, row_out, rows;
  if (which == 0) {          // K: rows = tokens, 128 elements each (16 chunks)
    rows = a.n_tok; row = c >> 4; col = (c & 15) * kDqChunk;
    src_row_len = kD; dst_row_len = kD; row_valid = kD; row_out = kD;
  } else {                   // V^T: rows = dims, tokens along the row; the
                             // destination row's columns past n_tok get zeros
    const int cpr = (a.dst_len + kDqChunk - 1) / kDqChunk;
    rows = kD; row = c / cpr; col = (c - row * cpr) * kDqChunk;
    src_row_len = a.src_len; dst_row_len = a.dst_len; row_valid = a.n_tok; row_out = a.dst_len;
  }
  if (row >= rows) return;
  const uint8_t* s = src + static_cast<int64_t>(row) * src_row_len + col;
  uint16_t* d = dst + static_cast<int64_t>(row) * dst_row_len + col;
  const int n = min(kDqChunk, row_valid - col);   // codes to convert (<= 0: none)
  const int n_out = min(kDqChunk, row_out - col);
  if (n == kDqChunk && (reinterpret_cast<uintptr_t>(s) & 7) == 0 &&
      (reinterpret_cast<uintptr_t>(d) & 15) == 0) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(s);
    u32x4 o;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // the hardware decode of e4m3 is exact (every code is an fp32 value)
      typedef float f32x2v __attribute__((ext_vector_type(2)));
      const f32x2v f01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x[m]), false);
      const f32x2v f23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(x[m]), true);
      o[2 * m] = pack_bf16x2(f01[0] * scale, f01[1] * scale);
      o[2 * m + 1] = pack_bf16x2(f23[0] * scale, f23[1] * scale);
    }
    *reinterpret_cast<u32x4*>(d) = o;
  } else {
    for (int j = 0; j < n_out; ++j) {
      const float v = j < n ? e4m3_to_f32(s[j]) * scale : 0.f;
      d[j] = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xFFFFu);
    }
  }
}

// int8 planes with a scale per token and head -> bf16 (code * scale, rounded).
// Same grid layout as dequant_kernel with 16-byte chunks: a K chunk is 16
// dims of one token (one scale), a V^T chunk 16 tokens of one dim row (16
// scales).
__global__ __launch_bounds__(256) void dequant_int8_kernel(const DequantArgs a) {
  const int i = blockIdx.y;
  const int h = blockIdx.z >> 1;
  const int which = blockIdx.z & 1;
  const int frame = a.frames != nullptr ? a.frames[i] : 0;
  const int64_t pl = static_cast<int64_t>(frame) * a.heads + h;
  const int8_t* src = reinterpret_cast<const int8_t*>(which ? a.src_v : a.src_k) + pl * a.src_len * kD;
  const float* sc = (which ? a.src_vs : a.src_ks) + pl * a.src_len;
  uint16_t* dst = (which ? a.dst_v : a.dst_k) +
                  (static_cast<int64_t>(i) * a.heads + h) * a.dst_len * kD;
  const int c = blockIdx.x * 256 + threadIdx.x;
  int row, col, src_row_len, dst_row_len, row_valid, row_out, rows;
  if (which == 0) {
    rows = a.n_tok; row = c >> 3; col = (c & 7) * 16;
    src_row_len = kD; dst_row_len = kD; row_valid = kD; row_out = kD;
  } else {                   // columns past n_tok of a V^T row get zeros
    const int cpr = (a.dst_len + 15) / 16;
    rows = kD; row = c / cpr; col = (c - row * cpr) * 16;
    src_row_len = a.src_len; dst_row_len = a.dst_len; row_valid = a.n_tok; row_out = a.dst_len;
  }
  if (row >= rows) return;
  const int8_t* s = src + static_cast<int64_t>(row) * src_row_len + col;
  uint16_t* d = dst + static_cast<int64_t>(row) * dst_row_len + col;
  const int n = min(16, row_valid - col);         // codes to convert (<= 0: none)
  const int n_out = min(16, row_out - col);
  for (int j = 0; j < n_out; j += 2) {
    const float s0 = j < n ? (which ? sc[col + j] : sc[row]) : 0.f;
    const float s1 = j + 1 < n ? (which ? sc[col + j + 1] : sc[row]) : 0.f;
    const float v0 = j < n ? static_cast<float>(s[j]) * s0 : 0.f;
    const float v1 = j + 1 < n ? static_cast<float>(s[j + 1]) * s1 : 0.f;
    const uint32_t w = pack_bf16x2(v0, v1);
    d[j] = static_cast<uint16_t>(w & 0xFFFFu);
    if (j + 1 < n_out) d[j + 1] = static_cast<uint16_t>(w >> 16);
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int64_t n16 = a.plane_bytes >> 4;
  const int64_t per_block = kGatherThreads * kChunksPerThread;
  dim3 grid(static_cast<unsigned>((n16 + per_block - 1) / per_block), a.n, 2);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kGatherThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  const int cb = a.int8 ? 16 : kDqChunk;   // bytes per chunk
  const int chunks_k = a.n_tok * (kD / cb);
  const int chunks_v = kD * ((a.dst_len + cb - 1) / cb);   // V^T rows up to the destination's length
  const int chunks = chunks_k > chunks_v ? chunks_k : chunks_v;
  dim3 grid((chunks + 255) / 256, a.n, a.heads * 2);
  if (a.int8)
    hipLaunchKernelGGL(dequant_int8_kernel, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
