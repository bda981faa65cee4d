// Top-K page selection.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §3: keep the K
// pages with the highest bounds; Implementation Step 2: a request with no
// more pages than the budget keeps all of them.  Ties go to the lower page
// index; the kept set is written in ascending page order, -1 padded.
//
// One workgroup per (request, kv-head) row.  Scores become order-preserving
// uint32 keys (-0 folded onto +0 first, so equal numbers get equal keys) and
// stay in registers, KPT consecutive pages per thread.  An MSB-first radix
// select with 8-bit digits (four passes, histograms in LDS) finds the key T
// of the k-th largest score and how many of the pages scoring exactly T
// still fit (need).  One block-wide exclusive scan of the packed per-thread
// counts (greater-than-T, equal-to-T) then gives every kept page its output
// slot: pages are visited in index order, so the lowest-index ties are kept
// and the output comes out ascending without a sort.
#include "common.h"
#include "launch.h"

namespace quest {
namespace {

__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u << 1) == 0) u = 0;  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

template <int BLOCK, int KPT>
__global__ void __launch_bounds__(BLOCK)
topk_kernel(const float* __restrict__ scores,
            const int32_t* __restrict__ seq_lens, int Hkv, int max_pages,
            int k, int32_t* __restrict__ sel) {
  constexpr int NW = BLOCK / kWave;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[NW];
  __shared__ uint32_t sh_prefix, sh_need;

  const int rowid = blockIdx.x;  // b * Hkv + g
  const int b = rowid / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int L = seq_lens[b];
  const int n = L > 0 ? min((L + kPageSize - 1) / kPageSize, max_pages) : 0;
  int32_t* out = sel + (int64_t)rowid * k;
  if (n <= k) {  // everything fits: keep all pages
    for (int i = tid; i < k; i += BLOCK) out[i] = i < n ? i : -1;
    return;
  }
  const float* s = scores + (int64_t)rowid * max_pages;
  uint32_t key[KPT];
  const int base = tid * KPT;
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = base + i < n ? score_key(s[base + i]) : 0u;

  uint32_t prefix = 0, mask = 0, need = (uint32_t)k;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += BLOCK) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (base + i < n && (key[i] & mask) == prefix)
        atomicAdd(&hist[(key[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (wid == 0) {
      // lane l owns digits 4l..4l+3; find the digit where the count of
      // larger-or-equal keys first reaches `need`, scanning from the top.
      uint32_t h[4], tot = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) { h[e] = hist[4 * lane + e]; tot += h[e]; }
      uint32_t incl = tot;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_down(incl, off, kWave);
        if (lane + off < kWave) incl += y;
      }
      uint32_t above = incl - tot;  // keys in digits above this lane's
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        if (above < need && above + h[e] >= need) {
          sh_prefix = prefix | ((uint32_t)(4 * lane + e) << shift);
          sh_need = need - above;
        }
        above += h[e];
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    need = sh_need;
    mask |= 255u << shift;
  }
  const uint32_t T = prefix;  // key of the k-th largest score

  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i < n) {
      gt += key[i] > T;
      eq += key[i] == T;
    }
  }
  const uint32_t packed = (gt << 16) | eq;  // counts < 65536 per block
  uint32_t incl = wave_incl_scan(packed, lane);
  if (lane == kWave - 1) wave_tot[wid] = incl;
  __syncthreads();
  uint32_t before = incl - packed;
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w < wid) before += wave_tot[w];
  uint32_t gt_before = before >> 16, eq_before = before & 0xffffu;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (base + i >= n) break;
    // slot = pages kept before this one; always < k (guarded all the same)
    if (key[i] > T) {
      const uint32_t slot = gt_before + min(eq_before, need);
      if (slot < (uint32_t)k) out[slot] = base + i;
      ++gt_before;
    } else if (key[i] == T) {
      const uint32_t slot = gt_before + eq_before;
      if (eq_before < need && slot < (uint32_t)k) out[slot] = base + i;
      ++eq_before;
    }
  }
}

template <int BLOCK, int KPT>
void launch_t(const quest_paged_kv& kv, const float* scores,
              const int32_t* seq_lens, int k, int32_t* sel,
              hipStream_t stream) {
  topk_kernel<BLOCK, KPT><<<kv.batch * kv.num_kv_heads, BLOCK, 0, stream>>>(
      scores, seq_lens, kv.num_kv_heads, kv.max_pages_per_seq, k, sel);
}

}  // namespace

hipError_t launch_topk(const quest_paged_kv& kv, const float* scores,
                       const int32_t* seq_lens, int k_pages, int32_t* sel,
                       hipStream_t stream) {
  const int mp = kv.max_pages_per_seq;
  if (mp <= 1024)       launch_t<256, 4>(kv, scores, seq_lens, k_pages, sel, stream);
  else if (mp <= 2048)  launch_t<256, 8>(kv, scores, seq_lens, k_pages, sel, stream);
  else if (mp <= 4096)  launch_t<512, 8>(kv, scores, seq_lens, k_pages, sel, stream);
  else if (mp <= 8192)  launch_t<1024, 8>(kv, scores, seq_lens, k_pages, sel, stream);
  else if (mp <= 16384) launch_t<1024, 16>(kv, scores, seq_lens, k_pages, sel, stream);
  else                  launch_t<1024, 32>(kv, scores, seq_lens, k_pages, sel, stream);
  return hipGetLastError();
}

}  // namespace quest
