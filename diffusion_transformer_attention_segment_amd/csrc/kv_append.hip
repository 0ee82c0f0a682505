// kv_append / text_append kernels: 3D RoPE on K, cache-plane stores of K and
// (transposed) V, bf16 or e4m3 + per-(frame, head) scales.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache",
// sections "How one segment is made" (RoPE split [16, 56, 56] over t, h, w)
// and "Writing the segment into memory" (the finished segment's K/V are
// stored); "The 4090 preset" (the cache is quantised once per segment).
//
// HBM-bound: per token and head the kernel reads 2 x 256 B of bf16 input and
// writes 2 x 256 B (bf16) or 2 x 128 B (e4m3) of cache.
#include "device_common.h"

namespace segattn {
namespace {

constexpr int kTileTok = 64;          // tokens per block tile
constexpr int kVtStride = kD + 8;     // LDS row stride (elements) of the V tile

// Rotate the 8 bf16 values of one 16-byte chunk (dims ch*8 .. ch*8+7) of a key
// at (t, h, w), in fp32, and return them rounded to bf16.
__device__ __forceinline__ void rotate_chunk(const u32x4& x, int ch, int t, int hh, int ww,
                                             const double* om, const int* ax, float* y) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint32_t wv = x[m];
    float a = __uint_as_float(wv << 16);
    float b = __uint_as_float(wv & 0xFFFF0000u);
    int pr = ch * 4 + m;
    int axis = ax[pr];
    int pos = axis == 0 ? t : (axis == 1 ? hh : ww);
    float c, s;
    rope_cos_sin(pos, om[pr], &c, &s);
    y[2 * m] = a * c - b * s;
    y[2 * m + 1] = a * s + b * c;
  }
}

__global__ __launch_bounds__(256) void append_bf16_kernel(const AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileTok * kVtStride];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * kTileTok;
  const int fr = blockIdx.y;
  const int h = blockIdx.z;
  const int H = a.heads;
  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();
  const int f = a.frame0 + fr;
  const size_t plane = static_cast<size_t>(a.plane_len) * kD;
  uint16_t* kdst = static_cast<uint16_t*>(a.k) + (static_cast<size_t>(f) * H + h) * plane;
  uint16_t* vdst = static_cast<uint16_t*>(a.v) + (static_cast<size_t>(f) * H + h) * plane;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int tok = c >> 4, ch = c & 15;
    const int p = p0 + tok;
    u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (p < a.n_tok) {
      const size_t in_off = (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
      kx = *reinterpret_cast<const u32x4*>(a.k_in + in_off);
      vx = *reinterpret_cast<const u32x4*>(a.v_in + in_off);
      u32x4 ky = kx;
      if (!a.is_text) {
        float y[8];
        rotate_chunk(kx, ch, f, p / a.rope.lat_w, p % a.rope.lat_w, om, ax, y);
#pragma unroll
        for (int m = 0; m < 4; ++m) ky[m] = pack_bf16x2(y[2 * m], y[2 * m + 1]);
      }
      *reinterpret_cast<u32x4*>(kdst + static_cast<size_t>(p) * kD + ch * 8) = ky;
    }
    *reinterpret_cast<u32x4*>(&vt[tok * kVtStride + ch * 8]) = vx;
  }
  __syncthreads();
  // transposed V: row d, tokens p0 + 8*tc .. +7
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int d = c >> 3, tc = c & 7;
    const int p = p0 + 8 * tc;
    if (p < a.plane_len) {
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t lo = vt[(8 * tc + 2 * m) * kVtStride + d];
        uint32_t hi = vt[(8 * tc + 2 * m + 1) * kVtStride + d];
        o[m] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(vdst + static_cast<size_t>(d) * a.plane_len + p) = o;
    }
  }
}

// ---------------------------------------------------------------- e4m3 path
// fp32 -> OCP e4m3fn code, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;
  if (a >= 448.0f) return 0x7Eu | sign;
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid 2^-9
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t ua = __float_as_uint(a);
    int e = static_cast<int>((ua >> 23) & 0xFF) - 127 + 7;
    uint32_t m3 = (ua >> 20) & 0x7u;
    const uint32_t rest = ua & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0u; ++e; }
    code = (static_cast<uint32_t>(e) << 3) | m3;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < static_cast<int>(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

constexpr int kFp8Threads = 512;

// One block per (frame, head) plane (or per head of the text slot): pass 1
// finds amax of the rotated K and of V, pass 2 quantises and stores.
__global__ __launch_bounds__(kFp8Threads) void append_fp8_kernel(const AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileTok * kVtStride];
  __shared__ double om[kD / 2];
  __shared__ int ax[kD / 2];
  __shared__ float red[kFp8Threads / 64];
  const int tid = threadIdx.x;
  const int fr = blockIdx.x;
  const int h = blockIdx.y;
  const int H = a.heads;
  if (tid < kD / 2) {
    int axis;
    om[tid] = rope_omega(tid, a.rope, &axis);
    ax[tid] = axis;
  }
  __syncthreads();
  const int f = a.frame0 + fr;
  const int n_chunks = a.n_tok * 16;
  float amk = 0.f, amv = 0.f;
  for (int c = tid; c < n_chunks; c += kFp8Threads) {
    const int p = c >> 4, ch = c & 15;
    const size_t in_off = (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(a.k_in + in_off);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(a.v_in + in_off);
    float y[8];
    if (!a.is_text) {
      rotate_chunk(kx, ch, f, p / a.rope.lat_w, p % a.rope.lat_w, om, ax, y);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        y[2 * m] = __uint_as_float(kx[m] << 16);
        y[2 * m + 1] = __uint_as_float(kx[m] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) amk = fmaxf(amk, fabsf(y[m]));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      amv = fmaxf(amv, fabsf(__uint_as_float(vx[m] << 16)));
      amv = fmaxf(amv, fabsf(__uint_as_float(vx[m] & 0xFFFF0000u)));
    }
  }
  amk = block_max(amk, red);
  amv = block_max(amv, red);
  const float ik = amk > 0.f ? 448.0f / amk : 1.0f;
  const float iv = amv > 0.f ? 448.0f / amv : 1.0f;
  if (tid == 0) {
    a.k_scale[static_cast<size_t>(f) * H + h] = amk > 0.f ? amk / 448.0f : 1.0f;
    a.v_scale[static_cast<size_t>(f) * H + h] = amv > 0.f ? amv / 448.0f : 1.0f;
  }
  const size_t plane = static_cast<size_t>(a.plane_len) * kD;
  uint8_t* kdst = static_cast<uint8_t*>(a.k) + (static_cast<size_t>(f) * H + h) * plane;
  uint8_t* vdst = static_cast<uint8_t*>(a.v) + (static_cast<size_t>(f) * H + h) * plane;
  for (int c = tid; c < n_chunks; c += kFp8Threads) {
    const int p = c >> 4, ch = c & 15;
    const size_t in_off = (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(a.k_in + in_off);
    float y[8];
    if (!a.is_text) {
      rotate_chunk(kx, ch, f, p / a.rope.lat_w, p % a.rope.lat_w, om, ax, y);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        y[2 * m] = __uint_as_float(kx[m] << 16);
        y[2 * m + 1] = __uint_as_float(kx[m] & 0xFFFF0000u);
      }
    }
    u32x2 o;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      o[m] = f32_to_e4m3(y[4 * m] * ik) | (f32_to_e4m3(y[4 * m + 1] * ik) << 8) |
             (f32_to_e4m3(y[4 * m + 2] * ik) << 16) | (f32_to_e4m3(y[4 * m + 3] * ik) << 24);
    }
    *reinterpret_cast<u32x2*>(kdst + static_cast<size_t>(p) * kD + ch * 8) = o;
  }
  // V: transpose through LDS, 64 tokens at a time; 16 tokens (16 bytes) per store.
  for (int p0 = 0; p0 < a.plane_len; p0 += kTileTok) {
    for (int c = tid; c < kTileTok * 16; c += kFp8Threads) {
      const int tok = c >> 4, ch = c & 15;
      const int p = p0 + tok;
      u32x4 vx = {0u, 0u, 0u, 0u};
      if (p < a.n_tok) {
        const size_t in_off = (static_cast<size_t>(fr * a.n_tok + p) * H + h) * kD + ch * 8;
        vx = *reinterpret_cast<const u32x4*>(a.v_in + in_off);
      }
      *reinterpret_cast<u32x4*>(&vt[tok * kVtStride + ch * 8]) = vx;
    }
    __syncthreads();
    {
      const int d = tid >> 2, tc = tid & 3;      // 128 rows x 4 chunks of 16 tokens
      const int p = p0 + 16 * tc;
      if (p < a.plane_len) {
        u32x4 o;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t word = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float x = bf16_to_f32(vt[(16 * tc + 4 * m + b) * kVtStride + d]);
            word |= f32_to_e4m3(x * iv) << (8 * b);
          }
          o[m] = word;
        }
        *reinterpret_cast<u32x4*>(vdst + static_cast<size_t>(d) * a.plane_len + p) = o;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s) {
  dim3 grid((a.plane_len + kTileTok - 1) / kTileTok, a.n_frames, a.heads);
  hipLaunchKernelGGL(append_bf16_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s) {
  dim3 grid(a.n_frames, a.heads);
  hipLaunchKernelGGL(append_fp8_kernel, grid, dim3(kFp8Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
