// Device helpers shared by the Quest kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 16;
constexpr int kWave = 64;

enum class DType : int { F16 = 0, BF16 = 1 };

// ---------------------------------------------------------------- storage

// Eight 16-bit values (one 16-byte load) widened to float32.  Both widenings
// are exact.
template <DType T>
__device__ __forceinline__ void widen8(const uint4& v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (T == DType::F16) {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xffffu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
    } else {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
}

// Total order on 16-bit floating-point encodings (fp16 and bf16 share the
// sign-magnitude layout): -inf < ... < -0 < +0 < ... < +inf as signed ints.
// The map is an involution on the encodings.
__device__ __forceinline__ int32_t ord16(uint32_t bits) {
  const int32_t s = (int32_t)(int16_t)(uint16_t)bits;
  return s >= 0 ? s : (s ^ 0x7fff);
}
__device__ __forceinline__ uint32_t unord16(int32_t k) {
  const int32_t s = k >= 0 ? k : (k ^ 0x7fff);
  return (uint32_t)(uint16_t)(int16_t)s;
}

// ------------------------------------------------------------ cross-lane

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                         0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the sum.  row_ror by 8, 4, 2, 1.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x122>(x);
  x += dpp<0x121>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) {
  return __shfl_xor(x, m, kWave);
}

// exp2 that maps (-inf) - (-inf) style inputs to 0 instead of NaN: callers
// pass a difference whose left side may be -inf.
__device__ __forceinline__ float exp2_or_zero(float a, float m) {
  return a == -INFINITY ? 0.f : exp2f(a - m);
}

}  // namespace quest
