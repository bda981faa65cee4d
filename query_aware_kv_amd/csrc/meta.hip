// Page metadata kernels: per-page, per-channel min/max of the keys.
//
// "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs", §1 (min/max
// equation): a page's box is the channelwise min and max of its keys.  Both
// are exact selections, done here on a total order of the 16-bit encodings
// (ord16), so fp16 and bf16 share one kernel and the result is bit-exact
// with -0 < +0.
//
// Layout: K tile of (page p, kv-head g) = 16 rows x 128 channels x 2 B =
// 4 KiB contiguous at ((p * Hkv + g) * 16) * 128 elements.  A wave covers
// one tile: lane = 16 * r + c reads 16 B (8 channels, chunk c) of rows
// r, r+4, r+8, r+12, so each load instruction reads 1 KiB contiguous.
#include <climits>

#include "common.h"
#include "launch.h"

namespace quest {
namespace {

// One wave per (request b, logical page j, kv-head g).
__global__ void __launch_bounds__(256)
meta_rebuild_kernel(const uint16_t* __restrict__ k_pool,
                    uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                    const int32_t* __restrict__ page_table,
                    const int32_t* __restrict__ seq_lens,
                    const int32_t* __restrict__ first_token, int Hkv,
                    int max_pages, int num_pool_pages, int S) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= max_pages * Hkv) return;
  const int j = unit / Hkv, g = unit - (unit / Hkv) * Hkv;
  const int L = seq_lens[b];
  const int v = min(S, L - j * S);  // valid tokens in page j
  if (v <= 0) return;
  const int f = first_token ? first_token[b] : 0;
  const int t0 = max(0, f - j * S);  // first token to fold
  if (t0 >= v) return;
  const int64_t p = page_table[(int64_t)b * max_pages + j];
  if (p < 0 || p >= num_pool_pages) return;  // not a pool page: nothing to read
  const int64_t tile = (p * Hkv + g) * ((int64_t)S * kHeadDim);
  const uint4* src = reinterpret_cast<const uint4*>(k_pool + tile);
  const int c = lane & 15, r = lane >> 4;

  int32_t mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { mn[e] = INT_MAX; mx[e] = INT_MIN; }
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // rows r + 4i of up to 32; v <= S bounds them
    const int t = r + 4 * i;
    if (t >= t0 && t < v) fold8(src[t * 16 + c], mn, mx);
  }
  // the four row groups (lanes c, c+16, c+32, c+48) meet
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t a, b;
    lane_pair<16>((uint32_t)mn[e], a, b);
    mn[e] = min((int32_t)a, (int32_t)b);
    lane_pair<16>((uint32_t)mx[e], a, b);
    mx[e] = max((int32_t)a, (int32_t)b);
    lane_pair<32>((uint32_t)mn[e], a, b);
    mn[e] = min((int32_t)a, (int32_t)b);
    lane_pair<32>((uint32_t)mx[e], a, b);
    mx[e] = max((int32_t)a, (int32_t)b);
  }
  const int64_t m = (p * Hkv + g) * kHeadDim + c * 8;
  uint4* dmin = reinterpret_cast<uint4*>(kmin + m);
  uint4* dmax = reinterpret_cast<uint4*>(kmax + m);
  if (t0 > 0) {  // entered mid-page: widen the existing box
    fold8(*dmin, mn, mx);
    fold8(*dmax, mn, mx);
  }
  if (r == 0) *dmin = pack8(mn);
  if (r == 1) *dmax = pack8(mx);
}

// One wave per (request b, kv-head g): write the appended token, fold it.
__global__ void __launch_bounds__(256)
meta_append_kernel(uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
                   uint16_t* __restrict__ kmin, uint16_t* __restrict__ kmax,
                   const int32_t* __restrict__ page_table,
                   const int32_t* __restrict__ seq_lens,
                   const uint16_t* __restrict__ k_new,
                   const uint16_t* __restrict__ v_new, int Hkv, int max_pages,
                   int num_pool_pages, int S) {
  const int b = blockIdx.y;
  const int g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (g >= Hkv || lane >= 32) return;
  const int L = seq_lens[b];
  if (L <= 0) return;
  const int pos = L - 1;
  const int j = pos / S, slot = pos - j * S;
  if (j >= max_pages) return;
  const int64_t p = page_table[(int64_t)b * max_pages + j];
  if (p < 0 || p >= num_pool_pages) return;
  const int c = lane & 15;
  const int64_t row = ((p * Hkv + g) * S + slot) * kHeadDim + c * 8;
  const int64_t src = ((int64_t)b * Hkv + g) * kHeadDim + c * 8;
  if (lane >= 16) {
    *reinterpret_cast<uint4*>(v_pool + row) =
        *reinterpret_cast<const uint4*>(v_new + src);
    return;
  }
  const uint4 x = *reinterpret_cast<const uint4*>(k_new + src);
  *reinterpret_cast<uint4*>(k_pool + row) = x;
  const int64_t m = (p * Hkv + g) * kHeadDim + c * 8;
  uint4* dmin = reinterpret_cast<uint4*>(kmin + m);
  uint4* dmax = reinterpret_cast<uint4*>(kmax + m);
  if (slot == 0) {
    *dmin = x;
    *dmax = x;
    return;
  }
  int32_t mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { mn[e] = INT_MAX; mx[e] = INT_MIN; }
  fold8(x, mn, mx);
  fold8(*dmin, mn, mx);
  fold8(*dmax, mn, mx);
  *dmin = pack8(mn);
  *dmax = pack8(mx);
}

}  // namespace

hipError_t launch_meta_rebuild(const quest_paged_kv& kv, const void* k_pool,
                               void* kmin, void* kmax,
                               const int32_t* page_table,
                               const int32_t* seq_lens,
                               const int32_t* first_token, hipStream_t stream) {
  const int64_t units = (int64_t)kv.max_pages_per_seq * kv.num_kv_heads;
  dim3 grid((unsigned)((units + 3) / 4), (unsigned)kv.batch);
  meta_rebuild_kernel<<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(k_pool), static_cast<uint16_t*>(kmin),
      static_cast<uint16_t*>(kmax), page_table, seq_lens, first_token,
      kv.num_kv_heads, kv.max_pages_per_seq, kv.num_pool_pages, kv.page_size);
  return hipGetLastError();
}

hipError_t launch_meta_append(const quest_paged_kv& kv, void* k_pool,
                              void* v_pool, void* kmin, void* kmax,
                              const int32_t* page_table,
                              const int32_t* seq_lens, const void* k_new,
                              const void* v_new, hipStream_t stream) {
  dim3 grid((unsigned)((kv.num_kv_heads + 3) / 4), (unsigned)kv.batch);
  meta_append_kernel<<<grid, 256, 0, stream>>>(
      static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
      static_cast<uint16_t*>(kmin), static_cast<uint16_t*>(kmax), page_table,
      seq_lens, static_cast<const uint16_t*>(k_new),
      static_cast<const uint16_t*>(v_new), kv.num_kv_heads,
      kv.max_pages_per_seq, kv.num_pool_pages, kv.page_size);
  return hipGetLastError();
}

}  // namespace quest
