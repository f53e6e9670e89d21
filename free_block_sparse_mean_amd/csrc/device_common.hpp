// Small device-side helpers shared by the HIP kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sol {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// 16-byte vector of the input dtype and its widening to float
template <typename T> struct Vec16;
template <> struct Vec16<__bf16> {
  static constexpr int kN = 8;
  typedef uint4 raw;
  __device__ static inline void to_float(const raw& r, float* f) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec16<float> {
  static constexpr int kN = 4;
  typedef float4 raw;
  __device__ static inline void to_float(const raw& r, float* f) {
    f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w;
  }
};

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// Reductions over the 4 lanes {l, l^16, l^32, l^48} (lanes that share l % 16)
// with the gfx950 permlane swaps: permlane16_swap(x, x) returns, in some
// order, the values of lane l and lane l^16, permlane32_swap those of l and
// l^32, so one VALU op per step replaces an LDS shuffle; both lanes of a pair
// combine the same two values in the same order, so they agree bit for bit.
__device__ inline float quad16_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float quad16_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// float -> bfloat16, round to nearest even (finite inputs)
__device__ inline __bf16 to_bf16(float f) { return (__bf16)f; }

}  // namespace sol
