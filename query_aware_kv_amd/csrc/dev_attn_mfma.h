// Decode attention of a GQA group (G >= 2 query heads sharing one kv-head)
// over 16-token tiles on the matrix cores.
//
// Same arithmetic contract as dev_attn.h (the attention equation of "Guide to
// Quest" and the paper summary's exact attention over the kept pages):
// float32 logits and softmax, float32 accumulation.  With G query heads per
// tile the step is a small contraction -- S = Q K^T is G x 16 over 128
// channels, O += P V is G x 128 over 16 tokens -- and on the VALU it costs
// G times the work of one head (the group-of-8 dense call runs 3x slower
// per byte than G = 1), so here both products run as 16 x 16 MFMAs with the
// heads padded to 16:
//
//   S^T (16 tokens x 16 heads) = K (16 x 128) . Q^T  : 4 x mfma 16x16x32 (f16/bf16)
//   O (16 heads x 128)        += P (16 x 16) . V     : 8 column blocks x 2 mfma 16x16x16
//
// The products of two fp16 (bf16) values are exact in float32, so S is the
// float32 dot product up to summation order.  P is float32; for the second
// product it is split into a high part (P rounded to the input type) and the
// rounded remainder, two MFMAs whose sum carries ~22 (fp16) or ~16 (bf16)
// bits of P, far below the 2e-3 output tolerance.
//
// Lane layouts (l = 16 g + j, g = l >> 4, j = l & 15; verified against a
// host matmul for all four instructions used):
//   mfma A operand: lane l holds row j, k = KPL*g .. KPL*g + KPL-1
//   mfma B operand: lane l holds col j, k = KPL*g .. KPL*g + KPL-1
//   mfma D        : lane l holds col j, rows 4g .. 4g+3
// Token rows are permuted so that both products line up without moving data
// between lanes: the K tile's A row j is token (j & 3) * 4 + (j >> 2), which
// puts S^T rows 4g+e (held by lane l) at token g + 4e -- exactly the tokens
// of the V rows this lane loads (the same V layout as dev_attn.h: token
// g + 4e, channels 8j .. 8j+7), and exactly the P entries the lane supplies
// as the A operand of the second product (row = head j, k = 4g + e).  V's
// column block b takes channel 8j + b for its column j, so lane (g, j) ends
// with O[head 4g + e][channel 8j + b], e < 4, b < 8.
#pragma once

#include "dev_attn.h"

namespace quest {

typedef _Float16 mf_h4 __attribute__((ext_vector_type(4)));
typedef _Float16 mf_h8 __attribute__((ext_vector_type(8)));
typedef short mf_s4 __attribute__((ext_vector_type(4)));
typedef __bf16 mf_b8 __attribute__((ext_vector_type(8)));
typedef float mf_f4 __attribute__((ext_vector_type(4)));

// S^T += A . B over 32 channels: A = 8 K values, B = 8 q values (16 B each).
template <DType T>
__device__ __forceinline__ mf_f4 mfma_qk(const uint4& a, const uint4& b, mf_f4 acc) {
  if constexpr (T == DType::F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf_h8, a),
                                                  __builtin_bit_cast(mf_h8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_b8, a),
                                                   __builtin_bit_cast(mf_b8, b), acc, 0, 0, 0);
}

// O += A . B over 16 tokens: A = 4 P values, B = 4 V values (two 16-bit
// values per dword).
template <DType T>
__device__ __forceinline__ mf_f4 mfma_pv(const uint2& a, const uint2& b, mf_f4 acc) {
  if constexpr (T == DType::F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mf_h4, a),
                                                 __builtin_bit_cast(mf_h4, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_s4, a),
                                                     __builtin_bit_cast(mf_s4, b), acc, 0, 0, 0);
}

// Round a finite float to the input type (round to nearest even), as bits.
template <DType T>
__device__ __forceinline__ uint32_t round16(float x) {
  if constexpr (T == DType::F16) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
  } else {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
}

template <DType T>
__device__ __forceinline__ float widen16(uint32_t h) {
  if constexpr (T == DType::F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else
    return __builtin_bit_cast(float, h << 16);
}

// Per-wave state: running max and sum of head j = lane & 15 (replicated over
// the four lane groups), and O[head 4g + e][channel 8j + b] in o[b][e].
struct MfmaAttnState {
  float m, l;
  mf_f4 o[8];
};

__device__ __forceinline__ void mfma_attn_init(MfmaAttnState& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] = mf_f4{0.f, 0.f, 0.f, 0.f};
}

// q as the B operand: head j (zero for j >= G), channels 32s + 8g .. +7.
template <int G>
__device__ __forceinline__ void mfma_load_q(const uint16_t* __restrict__ q, int64_t first_head,
                                            int lane, uint4 (&qb)[4]) {
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = j < G ? *reinterpret_cast<const uint4*>(q + (first_head + j) * kHeadDim + 32 * s + 8 * g)
                  : make_uint4(0, 0, 0, 0);
}

// The K tile as the A operand (row j = token (j & 3) * 4 + (j >> 2),
// channels 32s + 8g .. +7) and the V tile in the dev_attn.h layout (token
// g + 4e, channels 8j .. 8j+7), from the tile at element offset `tile`.
__device__ __forceinline__ void mfma_load_tile(const uint16_t* __restrict__ k_pool,
                                               const uint16_t* __restrict__ v_pool,
                                               int64_t tile, int lane, uint4 (&kx)[4],
                                               uint4 (&vx)[4]) {
  const int g = lane >> 4, j = lane & 15;
  const int krow = (j & 3) * 4 + (j >> 2);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    kx[s] = *reinterpret_cast<const uint4*>(k_pool + tile + krow * kHeadDim + 32 * s + 8 * g);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    vx[e] = *reinterpret_cast<const uint4*>(v_pool + tile + (g + 4 * e) * kHeadDim + 8 * j);
}

// Fold one 16-token tile (its first v tokens valid; v <= 0 changes nothing)
// into the wave's state.  qscale = sm_scale * log2(e) (exp2 domain).
template <DType T>
__device__ __forceinline__ void mfma_attn_page(MfmaAttnState& st, const uint4 (&qb)[4],
                                               const uint4 (&kx)[4], const uint4 (&vx)[4],
                                               int v, float qscale, int lane) {
  const int g = lane >> 4;
  mf_f4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) s = mfma_qk<T>(kx[i], qb[i], s);
  // logits of head j for tokens g + 4e
  float z[4];
  bool valid[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    valid[e] = g + 4 * e < v;
    z[e] = s[e] * qscale;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) mx = valid[e] ? fmaxf(mx, z[e]) : mx;
  mx = column4_max(mx);
  const float m_new = fmaxf(st.m, mx);
  const float alpha = exp2_or_zero(st.m, m_new);
  float p[4], ps = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = valid[e] ? exp2_hw(z[e] - m_new) : 0.f;
    ps += p[e];
  }
  ps = column4_sum(ps);
  st.l = st.l * alpha + ps;
  st.m = m_new;
  // rescale O rows (heads 4g + e) by their heads' alpha, held by lanes 4g + e
  float a_row[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) a_row[e] = __shfl(alpha, 4 * g + e, kWave);
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) st.o[b][e] *= a_row[e];
  // P as two A operands: rounded high part and rounded remainder
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = round16<T>(p[e]);
    lo[e] = round16<T>(p[e] - widen16<T>(hi[e]));
  }
  const uint2 a_hi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
  const uint2 a_lo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  // V column block b: channel 8j + b of tokens g + 4e, i.e. 16-bit element b
  // of vx[e].  Rows past the valid tokens may hold any bits (NaN included)
  // and become zeros first, as whole words, since 0 * NaN would not vanish
  // in the product.  Each B operand word pairs the same half of two rows'
  // words: one v_perm_b32 (byte selector 0x05040100 takes the low halves of
  // its second and first source, 0x07060302 the high halves).
  uint32_t vw[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vw[e][0] = valid[e] ? vx[e].x : 0u;
    vw[e][1] = valid[e] ? vx[e].y : 0u;
    vw[e][2] = valid[e] ? vx[e].z : 0u;
    vw[e][3] = valid[e] ? vx[e].w : 0u;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint32_t sel = (b & 1) ? 0x07060302u : 0x05040100u;
    const int wi = b >> 1;
    const uint2 vb = make_uint2(__builtin_amdgcn_perm(vw[1][wi], vw[0][wi], sel),
                                __builtin_amdgcn_perm(vw[3][wi], vw[2][wi], sel));
    st.o[b] = mfma_pv<T>(a_hi, vb, st.o[b]);
    st.o[b] = mfma_pv<T>(a_lo, vb, st.o[b]);
  }
}

// Publish the wave's state (heads h < G) to the workgroup's LDS in the
// dev_attn.h form, so attn_wg_partial combines the waves.  Caller syncs after.
template <int G, int WAVES>
__device__ __forceinline__ void mfma_attn_stage_wave(const MfmaAttnState& st,
                                                     AttnSmem<G, WAVES>& sm, int wid,
                                                     int lane) {
  const int g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int h = 4 * g + e;
    if (h < G) {
#pragma unroll
      for (int b = 0; b < 8; ++b) sm.o[wid][h][8 * j + b] = st.o[b][e];
    }
  }
  if (g == 0 && j < G) {
    sm.m[wid][j] = st.m;
    sm.l[wid][j] = st.l;
  }
}

}  // namespace quest
