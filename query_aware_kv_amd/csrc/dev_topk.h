// Top-K selection of one (request, kv-head) row by one workgroup.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §3: keep the k
// pages with the highest bounds; Implementation Step 2: a request with no
// more pages than the budget keeps all of them.  Ties go to the lower page
// index; the kept pages are written in ascending order, -1 padded.
//
// Scores become order-preserving uint32 keys (-0 folded onto +0 first, so
// equal numbers get equal keys), kept in VGPRs: KPT per thread, in segments
// of SEG consecutive pages -- thread t holds pages SEG*t .. SEG*t+SEG-1 of
// each stretch of SEG*BLOCK pages -- and optionally a short tail of TAIL
// pages per thread after the last stretch (topk_page).  SEG = 4 (the default) spreads a row just
// longer than 4*BLOCK pages over every wave, which the latency-bound
// launches want; SEG = KPT (one run per thread) needs one placement scan
// instead of KPT/4, which the many-row launches that share the CUs want.
// The block's min and max key fix how many leading bits all keys
// share; an MSB-first radix select then walks 8-bit digits of (key - min)
// from the highest differing bit, with histograms in LDS (double-buffered,
// so one barrier pair per pass), and stops as soon as the bin holding the
// k-th largest key is taken whole -- usually after one or two passes.  One
// block-wide exclusive scan of packed per-thread counts (above-threshold,
// at-threshold) per segment then gives every kept page its output slot:
// pages are visited in index order, so the lowest-index ties are the ones
// kept and the output is ascending without a sort.
#pragma once

#include "common.h"

namespace quest {

constexpr int kTopkSeg = 4;      // consecutive pages per segment (default)
constexpr int kTopkMaxSegs = 8;  // segments per thread (KPT <= 32)

template <int BLOCK>
struct TopkSmem {
  uint32_t hist[2][256];
  uint32_t red[2][BLOCK / kWave];                 // block min / max of the keys
  uint32_t scan[kTopkMaxSegs][BLOCK / kWave];     // per-wave totals of the final scan
  uint32_t prefix, need, count;
};

// Page of this thread's key i.  The first KPT - TAIL keys lie in segments
// of SEG consecutive pages (segment i / SEG, position i % SEG); the last
// TAIL keys are a run of TAIL consecutive pages per thread after every
// segment: pages SK*BLOCK + TAIL*t .. +TAIL-1 for thread t, SK = KPT - TAIL.
// A tail extends a row by TAIL*BLOCK pages at a fraction of the cost of a
// whole further segment (rows just past 2048 pages: 5 keys per thread
// instead of 8).
template <int BLOCK, int SEG, int SK = 0, int TAIL = 0>
__device__ __forceinline__ int topk_page(int i) {
  if (TAIL > 0 && i >= SK) return SK * BLOCK + (int)threadIdx.x * TAIL + (i - SK);
  return (i / SEG) * (BLOCK * SEG) + (int)threadIdx.x * SEG + i % SEG;
}

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u << 1) == 0) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wave min / max with DPP: rows by row_ror, then across rows by readlane.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x124, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x122, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x121, 0xf, 0xf, false));
  const uint32_t r0 = __builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = __builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = __builtin_amdgcn_readlane((int)x, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Load a thread's KPT scores (topk_page order); entries below `limit` are
// in bounds (limit = the row's length in the buffer), so callers can issue
// this before they know n.  Every load is issued, from an index clamped into
// the row, so they go out back to back; entries past `limit` hold anything
// and are never used (they are not pages of the row).  A 16-byte-aligned
// row whose length is a multiple of 4 is read with 16-byte loads.
// (TAIL: see topk_page; the tail keys are read one 4-byte load each.)
template <int BLOCK, int KPT, int SEG = kTopkSeg, int TAIL = 0>
__device__ __forceinline__ void topk_load(const float* __restrict__ s, int limit,
                                          float (&v)[KPT]) {
  constexpr int SK = KPT - TAIL;
  static_assert(SEG % 4 == 0 && SK % SEG == 0 && SK / SEG + (TAIL > 0) <= kTopkMaxSegs &&
                    TAIL >= 0 && TAIL < SEG,
                "whole 16-byte pieces and segments, a tail shorter than a segment");
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15u) == 0 && (limit & 3) == 0 &&
                   limit >= 4;
  if (vec) {  // row-uniform
#pragma unroll
    for (int i = 0; i < SK; i += 4) {
      const int b = min(topk_page<BLOCK, SEG, SK, TAIL>(i), limit - 4);  // each piece wholly in or out
      const float4 x = *reinterpret_cast<const float4*>(s + b);
      v[i] = x.x;
      v[i + 1] = x.y;
      v[i + 2] = x.z;
      v[i + 3] = x.w;
    }
#pragma unroll
    for (int i = SK; i < KPT; ++i) v[i] = s[min(topk_page<BLOCK, SEG, SK, TAIL>(i), limit - 1)];
  } else if (limit > 0) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = s[min(topk_page<BLOCK, SEG, SK, TAIL>(i), limit - 1)];
  } else {  // an empty row: nothing to read
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = 0.f;
  }
}

// The page-table entries of the same KPT pages, so that the kept pages' pool
// ids come out of the selection with no dependent load after it.
template <int BLOCK, int KPT, int SEG = kTopkSeg>
__device__ __forceinline__ void topk_load_table(const int32_t* __restrict__ pt_row,
                                                int limit, int32_t (&e)[KPT]) {
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = topk_page<BLOCK, SEG>(i);
    const int32_t x = limit > 0 ? pt_row[min(p, limit - 1)] : -1;
    e[i] = p < limit ? x : -1;
  }
}

// Select for one row.  The whole block (BLOCK threads) must call it.
//   v    : this thread's scores from topk_load with the same SEG (the row
//          has n <= BLOCK*KPT)
//   n_sink, n_local : when n > k, pages j < n_sink and j >= n - n_local are
//          kept whatever their scores ("Guide to Quest" §3: attention sinks
//          and the local window) and the other k - n_sink - n_local slots
//          go to the best remaining pages; needs n_sink + n_local <= k
//   out  : the k output slots are kept logical page indices ascending, then
//          -1; only slots w_lo <= slot < w_hi are written, slot s to
//          out[s - w_lo]
//   ent  : if non-null, this thread's page-table entries (topk_load_table);
//          then phys[s - w_lo] = the kept page's entry, -1 for the padding
//          (the pool page list used by attention), for the same slots
// Forced pages take no part in the radix select: it picks k - n_sink -
// n_local among the others, and the placement scan counts forced pages as
// kept, so the list stays ascending.
template <int BLOCK, int KPT, int SEG = kTopkSeg, int TAIL = 0>
__device__ __forceinline__ void topk_row(const float (&v)[KPT], int n, int k,
                         int n_sink, int n_local,
                         int32_t* __restrict__ out,
                         const int32_t (*ent)[KPT],
                         int32_t* __restrict__ phys, TopkSmem<BLOCK>& sm,
                         int w_lo = 0, int w_hi = 0x7fffffff) {
  constexpr int NW = BLOCK / kWave;
  constexpr int SK = KPT - TAIL;
  static_assert(NW >= 2, "one wave scans while the others clear");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  w_hi = min(w_hi, k);
  if (n <= k) {  // everything fits: keep every page
    for (int i = w_lo + tid; i < w_hi; i += BLOCK) {
      out[i - w_lo] = i < n ? i : -1;
      if (phys && i >= n) phys[i - w_lo] = -1;
    }
    if (phys) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int p = topk_page<BLOCK, SEG, SK, TAIL>(i);
        if (p < n && p >= w_lo && p < w_hi) phys[p - w_lo] = (*ent)[i];
      }
    }
    return;
  }
  // n > k >= n_sink + n_local: the forced ranges are disjoint and at least
  // one page competes.
  const int local0 = n - n_local;
  uint32_t key[KPT];
  bool forced[KPT], cand[KPT];
  uint32_t kmn = 0xffffffffu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = topk_page<BLOCK, SEG, SK, TAIL>(i);
    forced[i] = p < n && (p < n_sink || p >= local0);
    cand[i] = p < n && !forced[i];
    key[i] = cand[i] ? score_key(v[i]) : 0u;
    if (cand[i]) {
      kmn = min(kmn, key[i]);
      kmx = max(kmx, key[i]);
    }
  }
  kmn = wave_minmax_u32<false>(kmn);
  kmx = wave_minmax_u32<true>(kmx);
  if (lane == 0) {
    sm.red[0][wid] = kmn;
    sm.red[1][wid] = kmx;
  }
  for (int i = tid; i < 256; i += BLOCK) sm.hist[0][i] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmn = min(kmn, sm.red[0][w]);
    kmx = max(kmx, sm.red[1][w]);
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] -= kmn;  // rel key; invalid ones wrap, never read
  const uint32_t range = kmx - kmn;

  uint32_t prefix = 0, need = (uint32_t)(k - n_sink - n_local);
  const bool pick = need > 0;  // any competing slot at all
  int shift = 0;  // bits >= shift of the threshold are decided
  if (pick && range != 0) {
    const int bits = 32 - __clz(range);
    int hi = 32;                      // bits >= hi already decided
    shift = bits > 8 ? bits - 8 : 0;  // first digit: top 8 differing bits
    int buf = 0;
#pragma unroll 1
    for (;;) {
      // candidates: keys whose decided bits equal the prefix's
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool live = cand[i] && (hi >= 32 || (key[i] >> hi) == (prefix >> hi));
        if (live) atomicAdd(&sm.hist[buf][(key[i] >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wid == 0) {
        // lane l owns digits 255-4l down to 252-4l, so a prefix sum over the
        // lanes counts candidates from the top digit down; find the digit
        // whose bin holds the need-th largest candidate.
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) { h[e] = sm.hist[buf][255 - 4 * lane - e]; tot += h[e]; }
        uint32_t above = wave_scan_incl(tot) - tot;  // candidates in higher digits
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (above < need && above + h[e] >= need) {
            sm.prefix = (prefix & ~(0xffu << shift)) | ((uint32_t)(255 - 4 * lane - e) << shift);
            sm.need = need - above;
            sm.count = h[e];
          }
          above += h[e];
        }
      } else {
        for (int i = tid - kWave; i < 256; i += BLOCK - kWave) sm.hist[buf ^ 1][i] = 0;
      }
      __syncthreads();
      prefix = sm.prefix;
      need = sm.need;
      const uint32_t count = sm.count;
      if (count == need || shift == 0) break;  // bin taken whole, or exact
      hi = shift;
      shift = shift > 8 ? shift - 8 : 0;
      buf ^= 1;
    }
  }
  // Kept: forced pages, competing keys whose decided bits exceed the
  // threshold's, and the first `need` (in page order) whose decided bits
  // equal them.  "gt" counts the first two kinds.  Pages are ordered by
  // segment, then thread, then position: one packed count per segment (the
  // tail, if any, is the last segment, TAIL keys long).
  constexpr int NFULL = SK / SEG;
  constexpr int NSEG = NFULL + (TAIL > 0 ? 1 : 0);
  auto seg_len = [](int sg) { return sg < NFULL ? SEG : TAIL; };
  auto seg_key = [](int sg, int e) { return sg < NFULL ? sg * SEG + e : SK + e; };
  const uint32_t thr = shift >= 32 ? 0u : (prefix >> shift);
  uint32_t packed[NSEG], incl[NSEG];
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < SEG; ++e) {
      if (e >= seg_len(sg)) break;
      const int i = seg_key(sg, e);
      const uint32_t v = key[i] >> shift;
      gt += forced[i] || (pick && cand[i] && v > thr);
      eq += pick && cand[i] && v == thr;
    }
    packed[sg] = (gt << 16) | eq;  // both < 65536 (n <= 65535)
    incl[sg] = wave_scan_incl(packed[sg]);
    if (lane == kWave - 1) sm.scan[sg][wid] = incl[sg];
  }
  __syncthreads();
  uint32_t seg_base = 0;  // packed totals of the earlier segments
#pragma unroll
  for (int sg = 0; sg < NSEG; ++sg) {
    uint32_t before = incl[sg] - packed[sg] + seg_base;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wid) before += sm.scan[sg][w];
      seg_base += sm.scan[sg][w];
    }
    uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
#pragma unroll
    for (int e = 0; e < SEG; ++e) {
      if (e >= seg_len(sg)) break;
      const int i = seg_key(sg, e);
      const int page = topk_page<BLOCK, SEG, SK, TAIL>(i);
      if (page >= n) continue;
      const uint32_t v = key[i] >> shift;
      uint32_t slot = 0xffffffffu;
      if (forced[i] || (pick && cand[i] && v > thr)) {
        slot = gt_before + min(eq_before, need);
        ++gt_before;
      } else if (pick && cand[i] && v == thr) {
        if (eq_before < need) slot = gt_before + eq_before;
        ++eq_before;
      }
      if (slot - (uint32_t)w_lo < (uint32_t)(w_hi - w_lo)) {  // kept, in the window
        out[slot - w_lo] = page;
        if (phys) phys[slot - w_lo] = (*ent)[i];
      }
    }
  }
}

}  // namespace quest
