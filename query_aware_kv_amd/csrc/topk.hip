// quest_topk_pages(_ex): one workgroup per (request, kv-head) row runs the
// radix selection of dev_topk.h ("Guide to Quest", §3 and Implementation
// Step 2), with optional forced sink and local-window pages.
#include "dev_topk.h"
#include "launch.h"

namespace quest {
namespace {

// SEG: consecutive pages per thread and segment (dev_topk.h).
template <int BLOCK, int KPT, int SEG, int TAIL>
__global__ void __launch_bounds__(BLOCK)
topk_kernel(const float* __restrict__ scores,
            const int32_t* __restrict__ seq_lens, int Hkv, int max_pages,
            int k, int n_sink, int n_local, int page_size,
            int32_t* __restrict__ sel) {
  __shared__ TopkSmem<BLOCK> sm;
  const int rowid = blockIdx.x;  // b * Hkv + g
  const int b = rowid / Hkv;
  float v[KPT];  // issued together with the length load
  topk_load<BLOCK, KPT, SEG, TAIL>(scores + (int64_t)rowid * max_pages, max_pages, v);
  const int L = seq_lens[b];
  const int n = pages_of(L, page_size, max_pages);
  topk_row<BLOCK, KPT, SEG, TAIL>(v, n, k, n_sink, n_local, sel + (int64_t)rowid * k, nullptr,
                       nullptr, sm);
}

// 256-thread launches serve many rows: one run of KPT pages per thread;
// the wider ones serve few rows: segments of 4.
template <int BLOCK, int KPT, int TAIL = 0>
void launch_t(const quest_paged_kv& kv, const float* scores,
              const int32_t* seq_lens, int k, int n_sink, int n_local,
              int32_t* sel, hipStream_t stream) {
  constexpr int SEG = BLOCK <= 256 ? KPT : kTopkSeg;
  topk_kernel<BLOCK, KPT, SEG, TAIL><<<kv.batch * kv.num_kv_heads, BLOCK, 0, stream>>>(
      scores, seq_lens, kv.num_kv_heads, kv.max_pages_per_seq, k, n_sink, n_local,
      kv.page_size, sel);
}

}  // namespace

hipError_t launch_topk(const quest_paged_kv& kv, const float* scores,
                       const int32_t* seq_lens, int k_pages, int n_sink,
                       int n_local, int32_t* sel, hipStream_t stream) {
  const int mp = kv.max_pages_per_seq;
  // Up to 2048 pages: with few rows the selection's latency is the cost,
  // and 8 waves of 4 keys finish sooner than 4 waves of 8 (32 rows of 2048
  // pages: 5.0 vs 5.7 us); with many rows the workgroups share the CUs, and
  // the smaller ones go through faster (1024 rows: 16.9 vs 18.7 us).
  const bool few_rows = (int64_t)kv.batch * kv.num_kv_heads <= 256;
  if (mp <= 1024)       launch_t<256, 4>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 2048 && few_rows)
                        launch_t<512, 4>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 2560 && few_rows)  // 4 keys per thread + a tail of 1
                        launch_t<512, 5, 1>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 2048)  launch_t<256, 8>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 4096)  launch_t<512, 8>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 8192)  launch_t<1024, 8>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else if (mp <= 16384) launch_t<1024, 16>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  else                  launch_t<1024, 32>(kv, scores, seq_lens, k_pages, n_sink, n_local, sel, stream);
  return hipGetLastError();
}

}  // namespace quest
