// Top-K selection of one (request, kv-head) row by one workgroup.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §3: keep the k
// pages with the highest bounds; Implementation Step 2: a request with no
// more pages than the budget keeps all of them.  Ties go to the lower page
// index; the kept pages are written in ascending order, -1 padded.
//
// Scores become order-preserving uint32 keys (-0 folded onto +0 first, so
// equal numbers get equal keys), KPT consecutive pages per thread, kept in
// VGPRs.  The block's min and max key fix how many leading bits all keys
// share; an MSB-first radix select then walks 8-bit digits of (key - min)
// from the highest differing bit, with histograms in LDS (double-buffered,
// so one barrier pair per pass), and stops as soon as the bin holding the
// k-th largest key is taken whole -- usually after one or two passes.  One
// block-wide exclusive scan of packed per-thread counts (above-threshold,
// at-threshold) then gives every kept page its output slot: pages are
// visited in index order, so the lowest-index ties are the ones kept and the
// output is ascending without a sort.
#pragma once

#include "common.h"

namespace quest {

template <int BLOCK>
struct TopkSmem {
  uint32_t hist[2][256];
  uint32_t red[2][BLOCK / kWave];   // block min / max of the keys
  uint32_t scan[BLOCK / kWave];     // per-wave totals of the final scan
  uint32_t prefix, need, count;
};

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

// Load a thread's KPT consecutive scores; entries below `limit` are in
// bounds (limit = the row's length in the buffer), so callers can issue this
// before they know n.
template <int BLOCK, int KPT>
__device__ __forceinline__ void topk_load(const float* __restrict__ s, int limit,
                                          float (&v)[KPT]) {
  const int base = threadIdx.x * KPT;
#pragma unroll
  for (int i = 0; i < KPT; ++i) v[i] = base + i < limit ? s[base + i] : 0.f;
}

// The page-table entries of the same KPT pages, so that the kept pages' pool
// ids come out of the selection with no dependent load after it.
template <int BLOCK, int KPT>
__device__ __forceinline__ void topk_load_table(const int32_t* __restrict__ pt_row,
                                                int limit, int32_t (&e)[KPT]) {
  const int base = threadIdx.x * KPT;
#pragma unroll
  for (int i = 0; i < KPT; ++i) e[i] = base + i < limit ? pt_row[base + i] : -1;
}

// Select for one row.  The whole block (BLOCK threads) must call it.
//   v    : this thread's scores from topk_load (the row has n <= BLOCK*KPT)
//   out  : the k output slots are kept logical page indices ascending, then
//          -1; only slots lo <= slot < hi are written, slot s to out[s - lo]
//   ent  : if non-null, this thread's page-table entries (topk_load_table);
//          then phys[s - lo] = the kept page's entry, -1 for the padding (the
//          pool page list used by attention), for the same slots
template <int BLOCK, int KPT>
__device__ __forceinline__ void topk_row(const float (&v)[KPT], int n, int k,
                         int32_t* __restrict__ out,
                         const int32_t (*ent)[KPT],
                         int32_t* __restrict__ phys, TopkSmem<BLOCK>& sm,
                         int lo = 0, int hi = 0x7fffffff) {
  constexpr int NW = BLOCK / kWave;
  static_assert(NW >= 2, "one wave scans while the others clear");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  hi = min(hi, k);
  if (n <= k) {  // everything fits: keep every page
    for (int i = lo + tid; i < hi; i += BLOCK) {
      out[i - lo] = i < n ? i : -1;
      if (phys && i >= n) phys[i - lo] = -1;
    }
    if (phys) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int p = tid * KPT + i;
        if (p < n && p >= lo && p < hi) phys[p - lo] = (*ent)[i];
      }
    }
    return;
  }
  const int base = tid * KPT;
  uint32_t key[KPT];
  uint32_t kmn = 0xffffffffu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool ok = base + i < n;
    key[i] = ok ? score_key(v[i]) : 0u;
    if (ok) {
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

  uint32_t prefix = 0, need = (uint32_t)k;
  int shift = 0;  // bits >= shift of the threshold are decided
  if (range != 0) {
    const int bits = 32 - __clz(range);
    int hi = 32;                      // bits >= hi already decided
    shift = bits > 8 ? bits - 8 : 0;  // first digit: top 8 differing bits
    int buf = 0;
#pragma unroll 1
    for (;;) {
      // candidates: keys whose decided bits equal the prefix's
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool cand = base + i < n &&
                          (hi >= 32 || (key[i] >> hi) == (prefix >> hi));
        if (cand) atomicAdd(&sm.hist[buf][(key[i] >> shift) & 255u], 1u);
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
  // Kept: keys whose decided bits exceed the threshold's, plus the first
  // `need` (in page order) whose decided bits equal them.
  const uint32_t thr = shift >= 32 ? 0u : (prefix >> shift);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i < n) {
      const uint32_t v = key[i] >> shift;
      gt += v > thr;
      eq += v == thr;
    }
  }
  const uint32_t packed = (gt << 16) | eq;  // both < 65536 (n <= 65535)
  const uint32_t incl = wave_scan_incl(packed);
  if (lane == kWave - 1) sm.scan[wid] = incl;
  __syncthreads();
  uint32_t before = incl - packed;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wid) before += sm.scan[w];
  uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i >= n) break;
    const uint32_t v = key[i] >> shift;
    uint32_t slot = 0xffffffffu;
    if (v > thr) {
      slot = gt_before + min(eq_before, need);
      ++gt_before;
    } else if (v == thr) {
      if (eq_before < need) slot = gt_before + eq_before;
      ++eq_before;
    }
    if (slot - (uint32_t)lo < (uint32_t)(hi - lo)) {  // selected, in the window
      out[slot - lo] = base + i;
      if (phys) phys[slot - lo] = (*ent)[i];
    }
  }
}

}  // namespace quest
