// quest_union_pages: the union of a GQA group's per-query-head page
// selections ("Guide to Quest", Best Practices 2: the kv-head loads the
// union of its query heads' Top-K pages once, for all of them).
//
// One 256-thread workgroup per (request, kv-head): the G*k listed pages set
// bits of an LDS bitmap over the row's max_pages pages, then each thread
// counts the bits of its run of bitmap words, one block scan gives every
// thread its output offset, and the pages are written in ascending order
// (bit order), then -1 up to G*k.
#include "launch.h"

namespace quest {
namespace {

constexpr int kUnionThreads = 256;
constexpr int kUnionWords = kTopkMaxPages / 32;  // bitmap of up to 32768 pages

__global__ void __launch_bounds__(kUnionThreads)
union_kernel(const int32_t* __restrict__ sel_heads, int G, int k, int max_pages,
             int32_t* __restrict__ sel_union) {
  __shared__ uint32_t bm[kUnionWords];
  __shared__ uint32_t wsum[kUnionThreads / kWave];
  const int unit = blockIdx.x;  // b * Hkv + g
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int words = (max_pages + 31) / 32;
  for (int w = tid; w < words; w += kUnionThreads) bm[w] = 0u;
  __syncthreads();
  // rows g*G .. g*G+G-1 of [B][Hq][k] are contiguous: G*k entries from here
  const int32_t* src = sel_heads + (int64_t)unit * G * k;
  for (int i = tid; i < G * k; i += kUnionThreads) {
    const int p = src[i];
    if (p >= 0 && p < max_pages) atomicOr(&bm[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // thread t owns words [t*wpt, (t+1)*wpt)
  const int wpt = (words + kUnionThreads - 1) / kUnionThreads;
  const int w0 = tid * wpt;
  uint32_t cnt = 0;
  for (int w = w0; w < w0 + wpt && w < words; ++w) cnt += __popc(bm[w]);
  const uint32_t incl = wave_scan_incl(cnt);
  if (lane == kWave - 1) wsum[wid] = incl;
  __syncthreads();
  uint32_t off = incl - cnt;
  for (int w = 0; w < wid; ++w) off += wsum[w];
  uint32_t total = 0;
  for (int w = 0; w < kUnionThreads / kWave; ++w) total += wsum[w];
  int32_t* dst = sel_union + (int64_t)unit * G * k;
  for (int w = w0; w < w0 + wpt && w < words; ++w) {
    uint32_t bits = bm[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      dst[off++] = w * 32 + b;
    }
  }
  for (int i = (int)total + tid; i < G * k; i += kUnionThreads) dst[i] = -1;
}

}  // namespace

hipError_t launch_union(const quest_paged_kv& kv, const int32_t* sel_heads,
                        int k_pages, int32_t* sel_union, hipStream_t stream) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  union_kernel<<<kv.batch * kv.num_kv_heads, kUnionThreads, 0, stream>>>(
      sel_heads, G, k_pages, kv.max_pages_per_seq, sel_union);
  return hipGetLastError();
}

}  // namespace quest
