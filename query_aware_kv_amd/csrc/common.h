// Device helpers shared by the Quest kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quest {

constexpr int kHeadDim = 128;
// Kernels read pages as 16-token tiles: a page of S tokens (S = 16 or 32,
// the page sizes of "Guide to Quest", Best Practices 1) is S / 16 tiles.
constexpr int kTileRows = 16;
constexpr int kWave = 64;

__host__ __device__ constexpr bool page_size_supported(int S) { return S == 16 || S == 32; }

// Pages of a request of L tokens, clamped to the row's capacity.
__device__ __forceinline__ int pages_of(int L, int S, int max_pages) {
  return L > 0 ? min((L + S - 1) / S, max_pages) : 0;
}

enum class DType : int { F16 = 0, BF16 = 1 };

// ---------------------------------------------------------------- storage

// One 16-bit value of a packed word (half 0 = bits 0..15) widened to
// float32; for fp16 the conversion folds into v_fma_mix_f32 when the result
// feeds a multiply-add.
template <DType T>
__device__ __forceinline__ float widen_half(uint32_t w, int half) {
  if constexpr (T == DType::F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(half ? (w >> 16) : (w & 0xffffu)));
  else
    return __builtin_bit_cast(float, half ? (w & 0xffff0000u) : (w << 16));
}

// acc + a.lo * b.lo + a.hi * b.hi for two packed fp16 (bf16) pairs
// (v_dot2_f32_f16 / v_dot2_f32_bf16).  The products are exact in float32.
template <DType T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef short s2 __attribute__((ext_vector_type(2)));
  if constexpr (T == DType::F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), acc,
                                  false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s2, a), __builtin_bit_cast(s2, b),
                                           acc, false);
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

// Fold eight 16-bit values (one 16-byte piece) into running ord16 minima and
// maxima, and pack such keys back into eight 16-bit values.
__device__ __forceinline__ void fold8(const uint4& x, int32_t (&mn)[8],
                                      int32_t (&mx)[8]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t lo = ord16(w[i] & 0xffffu), hi = ord16(w[i] >> 16);
    mn[2 * i] = min(mn[2 * i], lo);
    mx[2 * i] = max(mx[2 * i], lo);
    mn[2 * i + 1] = min(mn[2 * i + 1], hi);
    mx[2 * i + 1] = max(mx[2 * i + 1], hi);
  }
}

__device__ __forceinline__ uint4 pack8(const int32_t (&k)[8]) {
  uint4 r;
  r.x = unord16(k[0]) | (unord16(k[1]) << 16);
  r.y = unord16(k[2]) | (unord16(k[3]) << 16);
  r.z = unord16(k[4]) | (unord16(k[5]) << 16);
  r.w = unord16(k[6]) | (unord16(k[7]) << 16);
  return r;
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

// Integer DPP move: lanes whose source is out of range (or masked off by
// row_mask) get 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row_shr by
// 1, 2, 4, 8 scans each 16-lane row, then row_bcast:15 and row_bcast:31
// carry the row totals into the rows above.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x) {
  x += dpp_u<0x111>(x);        // row_shr:1
  x += dpp_u<0x112>(x);        // row_shr:2
  x += dpp_u<0x114>(x);        // row_shr:4
  x += dpp_u<0x118>(x);        // row_shr:8
  x += dpp_u<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_u<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Broadcast of lane 63 (the total of an inclusive scan).
__device__ __forceinline__ uint32_t wave_last(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// The values of lane l and of its partner l ^ OFF: OFF = 16 pairs the rows
// of a wave two by two (v_permlane16_swap_b32), OFF = 32 pairs its halves
// (v_permlane32_swap_b32); one VALU instruction, no LDS round trip.  Both
// lanes of a pair receive the same two values in the same order, so a
// combine written in terms of (a, b) leaves both lanes bit-identical.
template <int OFF>
__device__ __forceinline__ void lane_pair(uint32_t x, uint32_t& a, uint32_t& b) {
  static_assert(OFF == 16 || OFF == 32, "row pairs or wave halves");
  if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
  }
}

template <int OFF>
__device__ __forceinline__ void lane_pair_f(float x, float& a, float& b) {
  uint32_t ua, ub;
  lane_pair<OFF>(__builtin_bit_cast(uint32_t, x), ua, ub);
  a = __builtin_bit_cast(float, ua);
  b = __builtin_bit_cast(float, ub);
}

// Max and sum of x over the lanes l, l ^ 16, l ^ 32, l ^ 48 (a column of
// the wave's four rows), identical on all four.
__device__ __forceinline__ float column4_max(float x) {
  float a, b;
  lane_pair_f<16>(x, a, b);
  lane_pair_f<32>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float column4_sum(float x) {
  float a, b;
  lane_pair_f<16>(x, a, b);
  lane_pair_f<32>(a + b, a, b);
  return a + b;
}

// 2^x on the transcendental unit (v_exp_f32, about 1 ulp), without the
// rescaling that keeps results below 2^-126 denormal: those flush to zero.
// Softmax weights that small are below float32 resolution of any sum they
// join (the largest weight of a row is 1).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 that maps (-inf) - (-inf) style inputs to 0 instead of NaN: callers
// pass a difference whose left side may be -inf.
__device__ __forceinline__ float exp2_or_zero(float a, float m) {
  return a == -INFINITY ? 0.f : exp2_hw(a - m);
}

}  // namespace quest
