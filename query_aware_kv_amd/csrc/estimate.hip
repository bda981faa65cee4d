// quest_estimate / quest_estimate_heads: the query-aware upper bound of every
// page of every (request, kv-head) row -- or of every query head
// ("Guide to Quest", §2 upper-bound inequality; Best Practices 2 for the
// per-head form; the arithmetic lives in dev_estimate.h).
//
// Work mapping: a 16-lane DPP row owns one kv-head g of one request and walks
// blocks of 4 consecutive pages, prefetching the next block's page ids while
// it scores the current one.  Rows of one wave take consecutive kv-heads,
// whose metadata sit next to each other in the pool.  When the kv-heads come
// in fours, the waves of a workgroup take the same four kv-heads over
// consecutive blocks: a wave still reads 1 KiB runs of bounds, and the
// workgroup's 16-byte score stores fill whole 64- or 128-byte pieces of each
// score row instead of pieces that 4 or 8 workgroups on different XCDs share.
#include "dev_estimate.h"
#include "launch.h"

namespace quest {
namespace {

constexpr int kRowsPerBlock = 16;  // 256 threads when kv-heads do not come in fours

// Extra arguments of the append mode (null otherwise).
struct EstAppend {
  uint16_t* k_pool;
  uint16_t* v_pool;
  const uint16_t* k_new;  // [B][Hkv][128]
  const uint16_t* v_new;
};

// PER_HEAD: scores hold one row per query head ([B][Hq][max_pages], head
// g * G + h) instead of one per kv-head with the group's sum.
// APPEND: first append token L_b - 1 (k_new / v_new) to its page and box,
// as quest_update_page_meta's append mode; the row that owns that page
// does it and scores the page with the updated box.
// quads: Hkv / 4 for the four-head mapping (workgroups of blockDim.x / 64
// waves), else 0.
template <DType T, int G, bool PER_HEAD, bool APPEND>
__global__ void __launch_bounds__(512)
estimate_kernel(const uint16_t* __restrict__ q,
                uint16_t* __restrict__ kmin,
                uint16_t* __restrict__ kmax,
                const int32_t* __restrict__ page_table,
                const int32_t* __restrict__ seq_lens,
                float* __restrict__ scores, int Hkv, int max_pages,
                int rows_per_head, int num_pool_pages, int page_size,
                int quads, EstAppend ap) {
  const int b = blockIdx.y;
  const int c = threadIdx.x & 15;
  int g, jb0;
  if (quads > 0) {
    // wave w: kv-heads 4 (x mod quads) .. +3, one per row, of first block
    // (x / quads) * waves + w
    const int waves = blockDim.x >> 6;
    jb0 = (int)(blockIdx.x / quads) * waves + (int)(threadIdx.x >> 6);
    g = (int)(blockIdx.x % quads) * 4 + (int)((threadIdx.x >> 4) & 3);
    if (jb0 >= rows_per_head) return;  // whole waves exit together
  } else {
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
    if (row >= rows_per_head * Hkv) return;  // whole 16-lane rows exit together
    g = row % Hkv;
    jb0 = row / Hkv;
  }
  const int32_t* pt_row = page_table + (int64_t)b * max_pages;
  float* srow = scores + ((int64_t)b * Hkv + g) * (PER_HEAD ? G : 1) * max_pages;
  // The length, the first table entries and q are independent loads.
  int ent[kEstPages];
  est_table(pt_row, max_pages, jb0 * kEstPages, ent);
  const int L = seq_lens[b];
  EstQ<G> qq;
  est_load_q<G>(q, ((int64_t)b * Hkv + g) * G, c, qq);
  const int n = pages_of(L, page_size, max_pages);
  // APPEND: the appended token's page, and the token itself, loaded up
  // front by the row that scores that page's block
  int jl = -1;
  uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
  if constexpr (APPEND) {
    jl = L > 0 ? (L - 1) / page_size : -1;
    const int jbl = jl >= 0 ? jl / kEstPages : -1;
    if (jbl >= jb0 && (jbl - jb0) % rows_per_head == 0) {
      const int64_t src = ((int64_t)b * Hkv + g) * kHeadDim + c * 8;
      kn = *reinterpret_cast<const uint4*>(ap.k_new + src);
      vn = *reinterpret_cast<const uint4*>(ap.v_new + src);
    }
  }

  for (int jb = jb0; jb * kEstPages < max_pages; jb += rows_per_head) {
    int pid[kEstPages];
    est_page_ids(ent, n, jb * kEstPages, num_pool_pages, pid);
    uint4 lo[kEstPages], hi[kEstPages];
    est_load_meta(kmin, kmax, pid, Hkv, g, c, lo, hi);
    if constexpr (APPEND) {
      const int u = jl - jb * kEstPages;  // the appended token's page in the block
      if (u >= 0 && u < kEstPages) {
        int64_t p = -1;
#pragma unroll
        for (int w = 0; w < kEstPages; ++w) if (w == u) p = pid[w];
        if (p >= 0)  // a pool page below n: L - 1 < n * page_size
          est_append(u, (L - 1) - jl * page_size, p, Hkv, g, c, page_size, kn, vn,
                     ap.k_pool, ap.v_pool, kmin, kmax, lo, hi);
      }
    }
    est_table(pt_row, max_pages, (jb + rows_per_head) * kEstPages, ent);  // prefetch
    if constexpr (PER_HEAD) {
      float s[G][kEstPages];
      est_score_heads<T, G>(qq, pid, lo, hi, s);
#pragma unroll
      for (int h = 0; h < G; ++h)
        est_store(srow + (int64_t)h * max_pages, jb * kEstPages, max_pages, c, pid, s[h]);
    } else {
      float s[kEstPages];
      est_score<T, G>(qq, pid, lo, hi, s);
      est_store(srow, jb * kEstPages, max_pages, c, pid, s);
    }
  }
}

template <DType T, int G, bool PER_HEAD, bool APPEND>
void launch_t(const quest_paged_kv& kv, const void* q, const void* kmin,
              const void* kmax, const int32_t* page_table,
              const int32_t* seq_lens, float* scores, const EstAppend& ap,
              hipStream_t stream) {
  const int Hkv = kv.num_kv_heads;
  const int blocks_per_head = (kv.max_pages_per_seq + kEstPages - 1) / kEstPages;
  // About 196608 16-lane rows (768 waves per CU over the launch, a few
  // 4-page blocks per row), never more rows per head than 4-page blocks.
  // Measured on the 32 x 32-head ragged batch: 24576 rows 156 us, 98304
  // 144 us, 196608 141 us, one block per row 145 us.  A single request
  // of 32 heads gets one block per row up to 24K pages.
  const int64_t target_rows = 196608;
  int64_t rph = target_rows / ((int64_t)Hkv * kv.batch);
  if (rph < 1) rph = 1;
  if (rph > blocks_per_head) rph = blocks_per_head;
  // Four-head mapping: 8 waves per workgroup (a full 128-byte line of 8
  // blocks' scores per kv-head) while that leaves at least 256 workgroups
  // and a row has more than 4 blocks, else 4.  A row that walks several
  // blocks strides by a multiple of the waves, so that every step of the
  // workgroup covers aligned blocks.  Measured on the 32-head LongChat
  // layer: 8.56 us against 9.44 us with 16 kv-heads of one block per
  // 4-wave workgroup, and 9.59 us with 16 waves.
  const int quads = Hkv % 4 == 0 ? Hkv / 4 : 0;
  int waves = 8;
  if (quads > 0 && (rph <= 4 || (int64_t)quads * ((rph + 7) / 8) * kv.batch < 256)) waves = 4;
  if (quads > 0 && rph < blocks_per_head && rph >= waves) rph -= rph % waves;
  const int64_t rows = rph * Hkv;
  dim3 grid(quads > 0 ? (unsigned)(quads * ((rph + waves - 1) / waves))
                      : (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock),
            (unsigned)kv.batch);
  const int threads = quads > 0 ? waves * kWave : kRowsPerBlock * 16;
  estimate_kernel<T, G, PER_HEAD, APPEND><<<grid, threads, 0, stream>>>(
      static_cast<const uint16_t*>(q),
      static_cast<uint16_t*>(const_cast<void*>(kmin)),
      static_cast<uint16_t*>(const_cast<void*>(kmax)), page_table, seq_lens, scores,
      Hkv, kv.max_pages_per_seq, (int)rph, kv.num_pool_pages, kv.page_size, quads, ap);
}

template <DType T, bool PER_HEAD, bool APPEND>
void dispatch_group(int G, const quest_paged_kv& kv, const void* q,
                    const void* kmin, const void* kmax,
                    const int32_t* page_table, const int32_t* seq_lens,
                    float* scores, const EstAppend& ap, hipStream_t stream) {
#define QUEST_EST(GG) \
  launch_t<T, GG, PER_HEAD, APPEND>(kv, q, kmin, kmax, page_table, seq_lens, scores, ap, stream)
  switch (G) {
    case 1: QUEST_EST(1); break;
    case 2: QUEST_EST(2); break;
    case 4: QUEST_EST(4); break;
    default: QUEST_EST(8); break;
  }
#undef QUEST_EST
}

}  // namespace

bool estimate_supported(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}

hipError_t launch_estimate(const quest_paged_kv& kv, const void* q,
                           const void* kmin, const void* kmax,
                           const int32_t* page_table, const int32_t* seq_lens,
                           float* scores, bool per_head, hipStream_t stream,
                           void* k_pool, void* v_pool, const void* k_new,
                           const void* v_new) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const EstAppend ap{static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                     static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new)};
  const bool append = k_new != nullptr;
#define QUEST_EST_D(TT, PH, AP) \
  dispatch_group<TT, PH, AP>(G, kv, q, kmin, kmax, page_table, seq_lens, scores, ap, stream)
  if (kv.dtype == QUEST_F16) {
    if (per_head) { if (append) QUEST_EST_D(DType::F16, true, true); else QUEST_EST_D(DType::F16, true, false); }
    else { if (append) QUEST_EST_D(DType::F16, false, true); else QUEST_EST_D(DType::F16, false, false); }
  } else {
    if (per_head) { if (append) QUEST_EST_D(DType::BF16, true, true); else QUEST_EST_D(DType::BF16, true, false); }
    else { if (append) QUEST_EST_D(DType::BF16, false, true); else QUEST_EST_D(DType::BF16, false, false); }
  }
#undef QUEST_EST_D
  return hipGetLastError();
}

}  // namespace quest
