// camera_attention: cross-attention of the segment's video tokens to the
// camera tokens of their frame chunk.
//
// Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache", section
// "The camera": a small cross-attention after each block reads one camera
// token per latent frame; with chunk size 1 the mask is block-diagonal (frame
// t sees only its own camera token), and the camera key/value projection is
// 2,048 x 128 (one 128-wide head, here shared by every query head, or one head
// per query head).
//
// HBM-bound: each (row, head) reads its 256-byte query and writes its
// 256-byte output; the chunk's <= 16 camera keys and values (a few KB per
// chunk) are read through the caches. Sixteen lanes own one (row, head), eight
// dims each (16-byte loads and stores); a dot product is eight FMAs and four
// butterfly shuffles inside the 16-lane group. The scores of the chunk stay
// in registers: max, exp2, sum, then the weighted values. With one key the
// weight is exactly 1 and the output is the camera value itself.
#include "device_common.h"

namespace segattn {
namespace {

constexpr int kCamThreads = 256;
constexpr int kGroups = kCamThreads / 16;   // (row, head) pairs per workgroup

__device__ __forceinline__ void unpack8(const uint4& u, float* x) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// sum over the 16 lanes of this lane's group
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kCamThreads) void camera_kernel(const CameraArgs a) {
  const int pair = blockIdx.x * kGroups + (threadIdx.x >> 4);
  const int lane = threadIdx.x & 15;
  const bool valid = pair < a.rows * a.heads;   // whole 16-lane groups agree
  const int row = valid ? pair / a.heads : 0;
  const int h = pair - (pair / a.heads) * a.heads;
  const int hk = a.kv_heads == 1 ? 0 : h;
  const int t = row / a.P;
  const int base = (t / a.chunk) * a.chunk;
  const int nk = min(a.chunk, a.n_cam - base);

  float q[8];
  unpack8(valid ? reinterpret_cast<const uint4*>(a.q + (static_cast<size_t>(row) * a.heads + h) * kD)[lane]
                : make_uint4(0u, 0u, 0u, 0u),
          q);
  float s[SA_MAX_CAMERA_CHUNK];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < SA_MAX_CAMERA_CHUNK; ++j) {
    s[j] = -INFINITY;
    if (j < nk) {
      float k[8];
      unpack8(reinterpret_cast<const uint4*>(
                  a.cam_k + (static_cast<size_t>(base + j) * a.kv_heads + hk) * kD)[lane], k);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf(q[i], k[i], d);
      s[j] = group_sum(d) * a.scale_log2;
      m = fmaxf(m, s[j]);
    }
  }
  float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SA_MAX_CAMERA_CHUNK; ++j) {
    if (j < nk) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m);
      float v[8];
      unpack8(reinterpret_cast<const uint4*>(
                  a.cam_v + (static_cast<size_t>(base + j) * a.kv_heads + hk) * kD)[lane], v);
      l += p;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(p, v[i], o[i]);
    }
  }
  if (!valid) return;
  const float inv = 1.0f / l;
  uint4 w;
  w.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  w.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  w.z = pack_bf16x2(o[4] * inv, o[5] * inv);
  w.w = pack_bf16x2(o[6] * inv, o[7] * inv);
  reinterpret_cast<uint4*>(a.out + (static_cast<size_t>(row) * a.heads + h) * kD)[lane] = w;
  if (a.lse != nullptr && lane == 0)
    a.lse[static_cast<size_t>(row) * a.heads + h] = (m + __log2f(l)) * 0.6931471805599453f;
}

}  // namespace

hipError_t launch_camera(const CameraArgs& a, hipStream_t s) {
  const int64_t pairs = static_cast<int64_t>(a.rows) * a.heads;
  hipLaunchKernelGGL(camera_kernel, dim3(static_cast<uint32_t>((pairs + kGroups - 1) / kGroups)),
                     dim3(kCamThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace segattn
