// Flash-decoding building blocks: online-softmax attention of G query heads
// over 16-token pages, and the merge of split partial results.
//
// "Quest: Query-Aware Sparsity for Efficient Long-Context LLM Inference"
// (paper summary), Summary, and "Guide to Quest", §3: exact softmax attention
// over the kept pages; the attention equation of "The Memory Bandwidth
// Bottleneck of Long-Context Decoding" (Guide to Quest) for the dense case.
//
// Lane = 16 r + c of a wave holds channels 8c..8c+7 of token rows r, r+4,
// r+8, r+12 of a page: each 16-byte load instruction reads 1 KiB contiguous
// and every byte is read by one lane.  A row's q.k is a DPP row reduction.
// Each row group r keeps its own online-softmax state over its tokens, so
// the page loop needs no cross-row traffic; row groups, waves and splits are
// combined afterwards with the usual rescaling.  Softmax runs in the exp2
// domain (logits scaled by sm_scale * log2 e); accumulation is float32.
// q.k is taken on packed 16-bit pairs with v_dot2 (exact products, float32
// sum) and scaled once per row.  Tokens past a request's end are masked by
// selection, never by multiplication, so unused slots may hold NaN.
#pragma once

#include "common.h"

namespace quest {

constexpr float kLog2e = 1.4426950408889634f;

template <int G>
struct AttnState {
  float m[G], l[G], o[G][8];
};

template <int G>
__device__ __forceinline__ void attn_init(AttnState<G>& st) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[h][e] = 0.f;
  }
}

// A lane's q: channels 8c..8c+7 of each of the G heads as four packed
// 16-bit pairs, and the logit scale (sm_scale * log2 e).
template <int G>
struct AttnQ {
  uint32_t w[G][4];
  float scale;
};

template <DType T, int G>
__device__ __forceinline__ void attn_load_q(const uint16_t* __restrict__ q,
                                            int64_t first_head, int c, float qscale,
                                            AttnQ<G>& qq) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + (first_head + h) * kHeadDim + c * 8);
    qq.w[h][0] = v.x;
    qq.w[h][1] = v.y;
    qq.w[h][2] = v.z;
    qq.w[h][3] = v.w;
  }
  qq.scale = qscale;
}

// Element offset of 16-token tile s of pool page p, kv-head g, for pages of
// SUB * 16 tokens ([P][Hkv][SUB*16][128]).
template <int SUB>
__device__ __forceinline__ int64_t attn_tile_offset(int64_t p, int Hkv, int g, int s) {
  return ((p * Hkv + g) * SUB + s) * (int64_t)(kTileRows * kHeadDim);
}

// 16-byte pieces of one 16-token tile (at element offset `tile`) for lane
// (r, c): rows r, r+4, r+8, r+12, channels 8c..8c+7.
__device__ __forceinline__ void attn_load_tile(const uint16_t* __restrict__ k_pool,
                                               const uint16_t* __restrict__ v_pool,
                                               int64_t tile, int r, int c,
                                               uint4 (&kx)[4], uint4 (&vx)[4]) {
  tile += c * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kx[i] = *reinterpret_cast<const uint4*>(k_pool + tile + (r + 4 * i) * kHeadDim);
    vx[i] = *reinterpret_cast<const uint4*>(v_pool + tile + (r + 4 * i) * kHeadDim);
  }
}

// Fold one 16-token tile (its first v tokens valid; v <= 0 changes nothing)
// into the row group's state.
template <DType T, int G>
__device__ __forceinline__ void attn_page(AttnState<G>& st, const AttnQ<G>& qq,
                                          const uint4 (&kx)[4], const uint4 (&vx)[4],
                                          int v, int r) {
  bool valid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) valid[i] = r + 4 * i < v;
  float z[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = dot2<T>(qq.w[h][0], kx[i].x, 0.f);
      acc = dot2<T>(qq.w[h][1], kx[i].y, acc);
      acc = dot2<T>(qq.w[h][2], kx[i].z, acc);
      acc = dot2<T>(qq.w[h][3], kx[i].w, acc);
      z[h][i] = row16_sum(acc) * qq.scale;
    }
  // V rows past the valid tokens become zeros (they may hold NaN), as
  // packed words, before widening
  uint32_t vw[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vw[i][0] = valid[i] ? vx[i].x : 0u;
    vw[i][1] = valid[i] ? vx[i].y : 0u;
    vw[i][2] = valid[i] ? vx[i].z : 0u;
    vw[i][3] = valid[i] ? vx[i].w : 0u;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = st.m[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = valid[i] ? fmaxf(mx, z[h][i]) : mx;
    const float alpha = exp2_or_zero(st.m[h], mx);
    float p[4], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = valid[i] ? exp2_hw(z[h][i] - mx) : 0.f;
      ps += p[i];
    }
    st.l[h] = st.l[h] * alpha + ps;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = st.o[h][e] * alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = fmaf(p[i], widen_half<T>(vw[i][e >> 1], e & 1), acc);
      st.o[h][e] = acc;
    }
    st.m[h] = mx;
  }
}

// Combine the four row groups of a wave (lanes c, c+16, c+32, c+48): two
// pairwise merges, each computed identically on both lanes of a pair.
template <int OFF, int G>
__device__ __forceinline__ void attn_combine_pair(AttnState<G>& st) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ma, mb, la, lb;
    lane_pair_f<OFF>(st.m[h], ma, mb);
    lane_pair_f<OFF>(st.l[h], la, lb);
    const float M = fmaxf(ma, mb);
    const float sa = exp2_or_zero(ma, M), sb = exp2_or_zero(mb, M);
    st.l[h] = la * sa + lb * sb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float oa, ob;
      lane_pair_f<OFF>(st.o[h][e], oa, ob);
      st.o[h][e] = oa * sa + ob * sb;
    }
    st.m[h] = M;
  }
}

template <int G>
__device__ __forceinline__ void attn_combine_rows(AttnState<G>& st) {
  attn_combine_pair<16>(st);
  attn_combine_pair<32>(st);
}

constexpr int kAttnWaves = 4;  // waves per attention workgroup (attn_split_kernel)

template <int G, int WAVES = kAttnWaves>
struct AttnSmem {
  float o[WAVES][G][kHeadDim];
  float m[WAVES][G], l[WAVES][G];
};

// Publish each wave's (row-combined) state to LDS.  Caller syncs after.
template <int G, int WAVES>
__device__ __forceinline__ void attn_stage_wave(const AttnState<G>& st,
                                                AttnSmem<G, WAVES>& sm, int wid, int r,
                                                int c) {
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.o[wid][h][c * 8 + e] = st.o[h][e];
      if (c == 0) {
        sm.m[wid][h] = st.m[h];
        sm.l[wid][h] = st.l[h];
      }
    }
  }
}

// The workgroup's combined (M, den, num[ch]) for head h, channel ch.
template <int G, int WAVES>
__device__ __forceinline__ void attn_wg_partial(const AttnSmem<G, WAVES>& sm, int h, int ch,
                                                float& M, float& den, float& num) {
  M = -INFINITY;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm.m[w][h]);
  den = 0.f;
  num = 0.f;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const float s = exp2_or_zero(sm.m[w][h], M);
    den += sm.l[w][h] * s;
    num += sm.o[w][h][ch] * s;
  }
}

struct MergeSmem {
  float m[kHeadDim], num[kHeadDim], den[kHeadDim];
};

// Fold the splits s = half, half + 2, ... of channel ch into a running
// (max, num, den), CHUNK splits per memory round trip.  Every load of a
// chunk is issued, from a split index clamped into range, so they go out
// back to back; splits past the end are masked afterwards.
template <int CHUNK>
__device__ __forceinline__ void merge_half(const float* __restrict__ o,
                                           const float* __restrict__ ml, int nsplit,
                                           int half, int ch, float& mr, float& num,
                                           float& den) {
  for (int s0 = half; s0 < nsplit; s0 += 2 * CHUNK) {
    float w[CHUNK], l[CHUNK], x[CHUNK];
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      const int sc = min(s0 + 2 * u, nsplit - 1);
      const float2 m_l = *reinterpret_cast<const float2*>(ml + 2 * sc);
      w[u] = m_l.x;
      l[u] = m_l.y;
      x[u] = o[(int64_t)sc * kHeadDim + ch];
    }
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      if (s0 + 2 * u >= nsplit) {
        w[u] = -INFINITY;
        l[u] = 0.f;
        x[u] = 0.f;
      }
    }
    float mc = mr;
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) mc = fmaxf(mc, w[u]);
    const float sc = exp2_or_zero(mr, mc);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      const float e = exp2_or_zero(w[u], mc);
      num += x[u] * e;
      den += l[u] * e;
    }
    mr = mc;
  }
}

// Fold the splits s = first, first + stride, ... of channel ch into a
// running (max, num, den), CHUNK splits per memory round trip, every load of
// a chunk issued from a clamped split index and masked afterwards.
template <int CHUNK>
__device__ __forceinline__ void merge_strided(const float* __restrict__ o,
                                              const float* __restrict__ ml, int nsplit,
                                              int first, int stride, int ch, float& mr,
                                              float& num, float& den) {
  for (int s0 = first; s0 < nsplit; s0 += stride * CHUNK) {
    float w[CHUNK], l[CHUNK], x[CHUNK];
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      const int sc = min(s0 + stride * u, nsplit - 1);
      const float2 m_l = *reinterpret_cast<const float2*>(ml + 2 * sc);
      w[u] = m_l.x;
      l[u] = m_l.y;
      x[u] = o[(int64_t)sc * kHeadDim + ch];
    }
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      if (s0 + stride * u >= nsplit) {
        w[u] = -INFINITY;
        l[u] = 0.f;
        x[u] = 0.f;
      }
    }
    float mc = mr;
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) mc = fmaxf(mc, w[u]);
    const float sc = exp2_or_zero(mr, mc);
    num *= sc;
    den *= sc;
#pragma unroll
    for (int u = 0; u < CHUNK; ++u) {
      const float e = exp2_or_zero(w[u], mc);
      num += x[u] * e;
      den += l[u] * e;
    }
    mr = mc;
  }
}

// Merge nsplit partials of one (request, query head) into out_row[128] with
// a 256-thread workgroup: partial s is (o[s*128 .. +128], ml[2s] = M,
// ml[2s+1] = den).  Thread (half, ch) folds channel ch of the splits of its
// parity with a running max (online softmax); the chunk matches the split
// count (4, 8 or 16 splits per half), so up to 32 splits take one memory
// round trip without loads to spare; the two halves then meet in LDS.
__device__ __forceinline__ void merge_splits(const float* __restrict__ o,
                                             const float* __restrict__ ml,
                                             int nsplit, float* __restrict__ out_row,
                                             MergeSmem& sm) {
  const int tid = threadIdx.x;
  const int ch = tid & (kHeadDim - 1), half = tid >> 7;
  float mr = -INFINITY, num = 0.f, den = 0.f;
  if (nsplit <= 8)
    merge_half<4>(o, ml, nsplit, half, ch, mr, num, den);
  else if (nsplit <= 16)
    merge_half<8>(o, ml, nsplit, half, ch, mr, num, den);
  else
    merge_half<16>(o, ml, nsplit, half, ch, mr, num, den);
  if (half == 1) {
    sm.m[ch] = mr;
    sm.num[ch] = num;
    sm.den[ch] = den;
  }
  __syncthreads();
  if (half == 0) {
    const float mo = sm.m[ch];
    const float M = fmaxf(mr, mo);
    const float sa = exp2_or_zero(mr, M), sb = exp2_or_zero(mo, M);
    const float d = den * sa + sm.den[ch] * sb;
    const float nm = num * sa + sm.num[ch] * sb;
    out_row[ch] = d > 0.f ? nm / d : 0.f;
  }
}

}  // namespace quest
