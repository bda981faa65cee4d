// Query-aware page estimate for a block of 4 consecutive pages of one
// (request, kv-head) row, computed by one 16-lane DPP row.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §2 (upper-bound
// inequality): a page's score is sum_i max(q_i * kmin_i, q_i * kmax_i); here
// unscaled, and a GQA group sums the bounds of its G query heads.
//
// Lane c of the row holds channels 8c..8c+7 of the G query heads (four
// packed 16-bit pairs per head) and reads 16 B of kmin and 16 B of kmax per
// page, so a page's 512 B of metadata is read once with 16-byte loads; the
// 16 partial sums of a page meet in a DPP row reduction.
//
// A box has kmin_i <= kmax_i in every channel, so max(q_i kmin_i, q_i kmax_i)
// is q_i kmax_i when q_i >= 0 and q_i kmin_i when q_i < 0 (for q_i = +-0 both
// products are zero).  The bound is therefore a dot product of q with the
// corner of the box that q's signs pick: a bit-select of the packed kmin /
// kmax words by a mask of q's sign bits, then v_dot2_f32_{f16,bf16}, which
// multiplies two pairs of 16-bit values and adds both products to a float32
// accumulator.  Products of two fp16 (or bf16) values are exact in float32;
// only the sum rounds.
#pragma once

#include "common.h"

namespace quest {

constexpr int kEstPages = 4;  // pages per 16-lane row per block

// One lane's share of the G query heads: channels 8c..8c+7 of head h as
// four words of two 16-bit values, and per word a mask that is 0xffff in
// each half whose q value has its sign bit set (negative, or -0).
template <int G>
struct EstQ {
  uint32_t w[G][4];
  uint32_t neg[G][4];
};

template <int G>
__device__ __forceinline__ void est_load_q(const uint16_t* __restrict__ q,
                                           int64_t first_head, int c, EstQ<G>& qq) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + (first_head + h) * kHeadDim + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qq.w[h][i] = w[i];
      qq.neg[h][i] = ((w[i] >> 15) & 0x00010001u) * 0xffffu;
    }
  }
}

// One lane's 8-channel part of head h's bound on a box (lo, hi).
template <DType T, int G>
__device__ __forceinline__ float est_part(const EstQ<G>& qq, int h, const uint4& lo,
                                          const uint4& hi, float acc) {
  const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t u[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = qq.neg[h][i];
    acc = dot2<T>(qq.w[h][i], (l[i] & m) | (u[i] & ~m), acc);
  }
  return acc;
}

// Page-table entries of logical pages j0..j0+3.  Entries up to max_pages
// are always in bounds, so they are read without waiting for the length.
__device__ __forceinline__ void est_table(const int32_t* __restrict__ pt_row,
                                          int max_pages, int j0,
                                          int (&ent)[kEstPages]) {
#pragma unroll
  for (int u = 0; u < kEstPages; ++u)
    ent[u] = j0 + u < max_pages ? pt_row[j0 + u] : -1;
}

// Pool pages of logical pages j0..j0+3 (-1 past n or outside the pool).
__device__ __forceinline__ void est_page_ids(const int (&ent)[kEstPages], int n,
                                             int j0, int num_pool_pages,
                                             int (&pid)[kEstPages]) {
#pragma unroll
  for (int u = 0; u < kEstPages; ++u) {
    const int p = ent[u];
    pid[u] = (j0 + u < n && p >= 0 && p < num_pool_pages) ? p : -1;
  }
}

__device__ __forceinline__ void est_load_meta(const uint16_t* __restrict__ kmin,
                                              const uint16_t* __restrict__ kmax,
                                              const int (&pid)[kEstPages], int Hkv,
                                              int g, int c, uint4 (&lo)[kEstPages],
                                              uint4 (&hi)[kEstPages]) {
#pragma unroll
  for (int u = 0; u < kEstPages; ++u) {
    if (pid[u] >= 0) {
      const int64_t m = ((int64_t)pid[u] * Hkv + g) * kHeadDim + c * 8;
      lo[u] = *reinterpret_cast<const uint4*>(kmin + m);
      hi[u] = *reinterpret_cast<const uint4*>(kmax + m);
    }
  }
}

// Bound of each of the 4 pages (every lane of the row gets all 4).
template <DType T, int G>
__device__ __forceinline__ void est_score(const EstQ<G>& qq,
                                          const int (&pid)[kEstPages],
                                          const uint4 (&lo)[kEstPages],
                                          const uint4 (&hi)[kEstPages],
                                          float (&s)[kEstPages]) {
#pragma unroll
  for (int u = 0; u < kEstPages; ++u) {
    float acc = 0.f;
    if (pid[u] >= 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc = est_part<T, G>(qq, h, lo[u], hi[u], acc);
    }
    s[u] = row16_sum(acc);
  }
}

// Append one token to page u of the block in registers and in memory, as
// quest_update_page_meta's append mode does ("Guide to Quest" §1: the box
// forms with its page; a token in slot 0 starts a new box): the row's 16
// lanes write the token's K and V row (8 channels each) and the updated box.
// `u` is uniform over the row; the loop keeps register indices constant.
__device__ __forceinline__ void est_append(int u, int slot, int64_t p, int Hkv, int g,
                                           int c, int S, const uint4& kn,
                                           const uint4& vn, uint16_t* __restrict__ k_pool,
                                           uint16_t* __restrict__ v_pool,
                                           uint16_t* __restrict__ kmin,
                                           uint16_t* __restrict__ kmax,
                                           uint4 (&lo)[kEstPages], uint4 (&hi)[kEstPages]) {
  const int64_t row = ((p * Hkv + g) * S + slot) * kHeadDim + c * 8;
  *reinterpret_cast<uint4*>(k_pool + row) = kn;
  *reinterpret_cast<uint4*>(v_pool + row) = vn;
#pragma unroll
  for (int w = 0; w < kEstPages; ++w) {
    if (w != u) continue;
    if (slot == 0) {
      lo[w] = kn;
      hi[w] = kn;
    } else {
      int32_t mn[8], mx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { mn[e] = 0x7fffffff; mx[e] = -0x7fffffff - 1; }
      fold8(kn, mn, mx);
      fold8(lo[w], mn, mx);
      fold8(hi[w], mn, mx);
      lo[w] = pack8(mn);
      hi[w] = pack8(mx);
    }
    const int64_t m = (p * Hkv + g) * kHeadDim + c * 8;
    *reinterpret_cast<uint4*>(kmin + m) = lo[w];
    *reinterpret_cast<uint4*>(kmax + m) = hi[w];
  }
}

// Per-query-head bounds of the 4 pages: s[h][u] for the G heads of the
// group, from one read of each box ("Guide to Quest", Best Practices 2).
template <DType T, int G>
__device__ __forceinline__ void est_score_heads(const EstQ<G>& qq,
                                                const int (&pid)[kEstPages],
                                                const uint4 (&lo)[kEstPages],
                                                const uint4 (&hi)[kEstPages],
                                                float (&s)[G][kEstPages]) {
#pragma unroll
  for (int u = 0; u < kEstPages; ++u) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float acc = pid[u] >= 0 ? est_part<T, G>(qq, h, lo[u], hi[u], 0.f) : 0.f;
      s[h][u] = row16_sum(acc);
    }
  }
}

// Store the 4 scores (-inf where there is no page): one 16-byte store by
// lane 0 of the row when the 4 slots are in the row and 16-byte aligned,
// else lanes 0..3 store one each.
__device__ __forceinline__ void est_store(float* __restrict__ srow, int j0,
                                          int max_pages, int c,
                                          const int (&pid)[kEstPages],
                                          const float (&s)[kEstPages]) {
  static_assert(kEstPages == 4, "one float4 per block");
  float w[kEstPages];
#pragma unroll
  for (int u = 0; u < kEstPages; ++u) w[u] = pid[u] >= 0 ? s[u] : -INFINITY;
  float* dst = srow + j0;
  if (j0 + kEstPages <= max_pages && (reinterpret_cast<uintptr_t>(dst) & 15u) == 0) {
    if (c == 0) *reinterpret_cast<float4*>(dst) = make_float4(w[0], w[1], w[2], w[3]);
  } else {
    // one predicated store per page, constant register indices only
#pragma unroll
    for (int u = 0; u < kEstPages; ++u)
      if (c == u && j0 + u < max_pages) dst[u] = w[u];
  }
}

}  // namespace quest
