// mfma_probe: throughput probes of the matrix pipes on the running device, for
// the measurement (libsegattn_probe.so, not part of the segment-attention ABI).
//
// Every probe keeps 8 independent 32x32 fp32 accumulators per wave (enough to
// hide the MFMA latency), runs workgroups of 8 waves (2 per SIMD, as the
// attention kernels), and writes one sum per thread so that nothing is
// removed. The operands decide the power drawn, and a power-limited chip
// clocks down with it, so the modes differ only in where the operands come
// from and how much they change:
//   0  bf16, constant register operands (1.0): the least toggling
//   1  bf16, random register operands, a different A for each MFMA
//   2  bf16, A read from LDS for every MFMA (one 16-byte ds_read per lane, as
//      the attention step reads its K or V^T operand, issued one iteration
//      ahead of its use), random contents
//   3  fp8 e4m3 (block-scaled 32x32x64 MFMA, unit scales), random register
//      operands, a different A for each MFMA
// FLOP per MFMA: 2 * 32 * 32 * 16 (bf16), 2 * 32 * 32 * 64 (fp8).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kChains = 8;
constexpr int kLdsWords = 65536 / 16;   // 64 KB of 16-byte words

template <int kMode>
__global__ __launch_bounds__(kThreads, 1) void mfma_bf16_probe(const u32x4* ops, int n_ops,
                                                               float* out, int iters) {
  __shared__ u32x4 lds[kMode == 2 ? kLdsWords : 1];
  const int tid = threadIdx.x, lane = tid & 63;
  if constexpr (kMode == 2) {
    for (int i = tid; i < kLdsWords; i += kThreads) lds[i] = ops[(i + blockIdx.x) % n_ops];
    __syncthreads();
  }
  bf16x8 a[kChains], b[2];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    const u32x4 x = kMode == 0 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                               : ops[(tid * 11 + j * 7 + blockIdx.x) % n_ops];
    a[j] = __builtin_bit_cast(bf16x8, x);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 x = kMode == 0 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                               : ops[(tid * 13 + j * 5 + 3 + blockIdx.x) % n_ops];
    b[j] = __builtin_bit_cast(bf16x8, x);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  if constexpr (kMode == 2) {   // A of iteration 0; each iteration reads the next one's
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      a[j] = __builtin_bit_cast(bf16x8, lds[(j * 64 + lane) & (kLdsWords - 1)]);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      const bf16x8 A = a[j];
      if constexpr (kMode == 2)
        a[j] = __builtin_bit_cast(
            bf16x8, lds[(((it + 1) * kChains + j) * 64 + lane) & (kLdsWords - 1)]);
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, b[j & 1], acc[j], 0, 0, 0);
    }
    // keeps the next iteration's reads in this one (the compiler would
    // otherwise move each read down to its use)
    if constexpr (kMode == 2) asm volatile("" ::: "memory");
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[static_cast<size_t>(blockIdx.x) * kThreads + tid] = s;
}

__global__ __launch_bounds__(kThreads, 1) void mfma_fp8_probe(const u32x4* ops, int n_ops,
                                                              float* out, int iters) {
  const int tid = threadIdx.x;
  i32x8 a[kChains], b[2];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    const u32x4 x = ops[(tid * 11 + j * 7 + blockIdx.x) % n_ops];
    const u32x4 y = ops[(tid * 11 + j * 7 + 1 + blockIdx.x) % n_ops];
    a[j] = i32x8{static_cast<int32_t>(x[0]), static_cast<int32_t>(x[1]), static_cast<int32_t>(x[2]),
                 static_cast<int32_t>(x[3]), static_cast<int32_t>(y[0]), static_cast<int32_t>(y[1]),
                 static_cast<int32_t>(y[2]), static_cast<int32_t>(y[3])};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 x = ops[(tid * 13 + j * 5 + 3 + blockIdx.x) % n_ops];
    const u32x4 y = ops[(tid * 13 + j * 5 + 4 + blockIdx.x) % n_ops];
    b[j] = i32x8{static_cast<int32_t>(x[0]), static_cast<int32_t>(x[1]), static_cast<int32_t>(x[2]),
                 static_cast<int32_t>(x[3]), static_cast<int32_t>(y[0]), static_cast<int32_t>(y[1]),
                 static_cast<int32_t>(y[2]), static_cast<int32_t>(y[3])};
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[j & 1], acc[j], 0, 0, 0, 127,
                                                               0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[static_cast<size_t>(blockIdx.x) * kThreads + tid] = s;
}

}  // namespace

// Launches probe `mode` (0-3 above) on `stream`: `grid` workgroups of 512
// threads, `iters` iterations of 8 MFMAs per wave. ops: device array of n_ops
// 16-byte words of operand bits (random finite bf16 pairs for modes 1-2;
// e4m3 bytes without NaN codes for mode 3; unused by mode 0 but must hold at
// least one word); out: device float [grid * 512]. Returns 0, -1 for bad
// arguments (nothing launched), or the HIP error of the launch.
extern "C" int sa_probe_mfma(int mode, const void* ops, int n_ops, float* out, int grid, int iters,
                             void* stream) {
  if (mode < 0 || mode > 3 || ops == nullptr || n_ops < 1 || out == nullptr || grid < 1 ||
      iters < 1)
    return -1;
  const u32x4* o = static_cast<const u32x4*>(ops);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_bf16_probe<0>, dim3(grid), dim3(kThreads), 0, s, o, n_ops, out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_bf16_probe<1>, dim3(grid), dim3(kThreads), 0, s, o, n_ops, out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_bf16_probe<2>, dim3(grid), dim3(kThreads), 0, s, o, n_ops, out, iters); break;
    default: hipLaunchKernelGGL(mfma_fp8_probe, dim3(grid), dim3(kThreads), 0, s, o, n_ops, out, iters); break;
  }
  return static_cast<int>(hipGetLastError());
}
