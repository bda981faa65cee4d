// Query-aware page estimate.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §2 (upper-bound
// inequality): a page's score is sum_i max(q_i * kmin_i, q_i * kmax_i); here
// unscaled, and a GQA group sums the bounds of its G query heads.
//
// Work mapping: a "row" of 16 lanes (one DPP row) owns one kv-head g of one
// request and walks blocks of 4 consecutive logical pages; lane c of the row
// holds channels 8c..8c+7 of the G query heads in registers (G*8 floats) and
// reads 16 B of kmin and 16 B of kmax per page, so each page's 512 B of
// metadata is read exactly once with 16-byte loads.  Rows of one wave take
// consecutive kv-heads, which sit next to each other in the metadata.  The
// 16 partial sums of a page meet through a DPP row reduction.  Products of
// two fp16 (or bf16) values are exact in float32; only the sum rounds.
#include "common.h"
#include "launch.h"

namespace quest {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads
constexpr int kPagesPerIter = 4;

template <DType T, int G>
__global__ void __launch_bounds__(256)
estimate_kernel(const uint16_t* __restrict__ q,
                const uint16_t* __restrict__ kmin,
                const uint16_t* __restrict__ kmax,
                const int32_t* __restrict__ page_table,
                const int32_t* __restrict__ seq_lens,
                float* __restrict__ scores, int Hkv, int max_pages,
                int rows_per_head, int num_pool_pages) {
  const int b = blockIdx.y;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (row >= rows_per_head * Hkv) return;  // whole 16-lane rows exit together
  const int g = row % Hkv;
  const int jb0 = row / Hkv;
  const int L = seq_lens[b];
  const int n = L > 0 ? min((L + kPageSize - 1) / kPageSize, max_pages) : 0;

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t off = (((int64_t)b * Hkv + g) * G + h) * kHeadDim + c * 8;
    widen8<T>(*reinterpret_cast<const uint4*>(q + off), qf[h]);
  }
  const int32_t* pt = page_table + (int64_t)b * max_pages;
  float* srow = scores + ((int64_t)b * Hkv + g) * max_pages;

  auto load_ids = [&](int jb, int (&pid)[kPagesPerIter]) {
#pragma unroll
    for (int u = 0; u < kPagesPerIter; ++u) {
      const int j = jb * kPagesPerIter + u;
      pid[u] = j < n ? pt[j] : -1;
      if (pid[u] >= num_pool_pages) pid[u] = -1;  // not a pool page
    }
  };

  int pid[kPagesPerIter];
  load_ids(jb0, pid);
  for (int jb = jb0; jb * kPagesPerIter < max_pages; jb += rows_per_head) {
    uint4 lo[kPagesPerIter], hi[kPagesPerIter];
#pragma unroll
    for (int u = 0; u < kPagesPerIter; ++u) {
      if (pid[u] >= 0) {
        const int64_t m = ((int64_t)pid[u] * Hkv + g) * kHeadDim + c * 8;
        lo[u] = *reinterpret_cast<const uint4*>(kmin + m);
        hi[u] = *reinterpret_cast<const uint4*>(kmax + m);
      }
    }
    int cur[kPagesPerIter];
#pragma unroll
    for (int u = 0; u < kPagesPerIter; ++u) cur[u] = pid[u];
    load_ids(jb + rows_per_head, pid);  // prefetch the next block's page ids

    float s[kPagesPerIter];
#pragma unroll
    for (int u = 0; u < kPagesPerIter; ++u) {
      float acc = 0.f;
      if (cur[u] >= 0) {
        float a[8], z[8];
        widen8<T>(lo[u], a);
        widen8<T>(hi[u], z);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc += fmaxf(qf[h][e] * a[e], qf[h][e] * z[e]);
      }
      s[u] = row16_sum(acc);
    }
    if (c < kPagesPerIter) {
      const int j = jb * kPagesPerIter + c;
      const float v = c == 0 ? s[0] : c == 1 ? s[1] : c == 2 ? s[2] : s[3];
      const int id = c == 0 ? cur[0] : c == 1 ? cur[1] : c == 2 ? cur[2] : cur[3];
      if (j < max_pages) srow[j] = id >= 0 ? v : -INFINITY;  // id < 0: j >= n
    }
  }
}

template <DType T, int G>
void launch_t(const quest_paged_kv& kv, const void* q, const void* kmin,
              const void* kmax, const int32_t* page_table,
              const int32_t* seq_lens, float* scores, hipStream_t stream) {
  const int Hkv = kv.num_kv_heads;
  const int blocks_per_head =
      (kv.max_pages_per_seq + kPagesPerIter - 1) / kPagesPerIter;
  // Enough rows to keep ~24 waves per CU busy on 256 CUs, and never more
  // rows per head than 4-page blocks.
  const int64_t target_rows = 24576;
  int64_t rph = target_rows / ((int64_t)Hkv * kv.batch);
  if (rph < 1) rph = 1;
  if (rph > blocks_per_head) rph = blocks_per_head;
  const int64_t rows = rph * Hkv;
  dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock),
            (unsigned)kv.batch);
  estimate_kernel<T, G><<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kmin),
      static_cast<const uint16_t*>(kmax), page_table, seq_lens, scores, Hkv,
      kv.max_pages_per_seq, (int)rph, kv.num_pool_pages);
}

template <DType T>
bool dispatch_group(int G, const quest_paged_kv& kv, const void* q,
                    const void* kmin, const void* kmax,
                    const int32_t* page_table, const int32_t* seq_lens,
                    float* scores, hipStream_t stream) {
  switch (G) {
    case 1: launch_t<T, 1>(kv, q, kmin, kmax, page_table, seq_lens, scores, stream); return true;
    case 2: launch_t<T, 2>(kv, q, kmin, kmax, page_table, seq_lens, scores, stream); return true;
    case 4: launch_t<T, 4>(kv, q, kmin, kmax, page_table, seq_lens, scores, stream); return true;
    case 8: launch_t<T, 8>(kv, q, kmin, kmax, page_table, seq_lens, scores, stream); return true;
    default: return false;
  }
}

}  // namespace

bool estimate_supported(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}

hipError_t launch_estimate(const quest_paged_kv& kv, const void* q,
                           const void* kmin, const void* kmax,
                           const int32_t* page_table, const int32_t* seq_lens,
                           float* scores, hipStream_t stream) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  if (kv.dtype == QUEST_F16)
    dispatch_group<DType::F16>(G, kv, q, kmin, kmax, page_table, seq_lens, scores, stream);
  else
    dispatch_group<DType::BF16>(G, kv, q, kmin, kmax, page_table, seq_lens, scores, stream);
  return hipGetLastError();
}

}  // namespace quest
