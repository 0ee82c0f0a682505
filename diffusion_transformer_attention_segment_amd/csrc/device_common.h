// Device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace segattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 for two values, packed low/high
// (hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Frequency of rotation pair `pair` (dims 2*pair, 2*pair+1) of the 128-dim
// head under a [s0, s1, s2] split: theta^(-2j/n) for pair j of its band, in
// fp64. Also returns which axis (0 = t, 1 = h, 2 = w) drives the pair.
__device__ __forceinline__ double rope_omega(int pair, const RopeParams& r, int* axis) {
  int d = 2 * pair;
  int j, n;
  if (d < r.split0) {
    *axis = 0; j = pair; n = r.split0;
  } else if (d < r.split0 + r.split1) {
    *axis = 1; j = (d - r.split0) / 2; n = r.split1;
  } else {
    *axis = 2; j = (d - r.split0 - r.split1) / 2; n = r.split2;
  }
  return exp2(-2.0 * j / n * r.log2_theta);
}

// cos/sin of pos * omega: the angle is formed and reduced modulo 2*pi in
// fp64, then evaluated in fp32, so the rotation error stays near one fp32 ulp
// for positions in the tens of thousands.
__device__ __forceinline__ void rope_cos_sin(int pos, double omega, float* c, float* s) {
  const double kTwoPiHi = 6.283185307179586;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double kInvTwoPi = 0.15915494309189535;
  double ang = static_cast<double>(pos) * omega;
  double k = rint(ang * kInvTwoPi);
  double red = fma(-k, kTwoPiHi, ang);
  red = fma(-k, kTwoPiLo, red);
  sincosf(static_cast<float>(red), s, c);
}

}  // namespace segattn
