// quest_topk_sparse_decode_attn: Top-K selection and sparse attention of a
// decode step in one launch (plus the split merge), with no hand-off between
// workgroups.
//
// The steps are those of quest_topk_pages and quest_sparse_decode_attn
// ("Guide to Quest" §3 and Implementation Step 2; the paper summary's exact
// attention over the kept pages); the arithmetic is dev_topk.h and
// dev_attn.h.  What changes is where the selection lives: every attention
// workgroup of a (request, kv-head) row reads the row's scores (a few KiB)
// and runs the row's Top-K itself, keeping the kept-page list in LDS.  All
// workgroups of a row compute the identical list (the selection is exact and
// deterministic), so none has to wait for another; each then writes its own
// slice of sel_pages and attends over the same slice of the list.  This
// removes a launch and the global round trip of the selection.
//
// Workgroups have 8 waves (one slice of 8 * PPW pages): the selection is
// repeated once per workgroup, so half as many workgroups as with 4 waves
// halves that repeated work while the same number of waves stream K/V.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "dev_attn.h"
#include "dev_attn_mfma.h"
#include "dev_topk.h"
#include "launch.h"

namespace quest {
namespace {

constexpr int kTaWaves = 8;
constexpr int kTaThreads = kTaWaves * kWave;

template <DType T, int G, int KPT, int PPW, int SUB, int TAIL>
__global__ void __launch_bounds__(kTaThreads)
topk_attn_kernel(const uint16_t* __restrict__ q,
                 const uint16_t* __restrict__ k_pool,
                 const uint16_t* __restrict__ v_pool,
                 const int32_t* __restrict__ page_table,
                 const int32_t* __restrict__ seq_lens,
                 const float* __restrict__ scores, int k, int n_sink,
                 int n_local, int Hkv,
                 int max_pages, int num_pool_pages, float qscale,
                 int32_t* __restrict__ sel, float* __restrict__ out,
                 float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ union {
    TopkSmem<kTaThreads> topk;
    AttnSmem<G, kTaWaves> attn;
  } sm;
  // This workgroup's slice of the row's selection.
  __shared__ int32_t kept[kTaWaves * PPW];
  const int unit = blockIdx.y;       // b * Hkv + g
  const int b = unit / Hkv, g = unit - (unit / Hkv) * Hkv;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c = lane & 15, r = lane >> 4;

  // Scores, the length and q are independent loads.
  float v[KPT];
  topk_load<kTaThreads, KPT, kTopkSeg, TAIL>(scores + (int64_t)unit * max_pages, max_pages,
                                             v);
  const int L = seq_lens[b];
  // q: packed words of one head (VALU path), the MFMA operand for a group
  AttnQ<G> qf;
  uint4 qb[4];
  if constexpr (G >= 2)
    mfma_load_q<G>(q, (int64_t)unit * G, lane, qb);
  else
    attn_load_q<T, G>(q, (int64_t)unit * G, c, qscale, qf);
  constexpr int S = SUB * kTileRows;
  const int n = pages_of(L, S, max_pages);
  const int s0 = split * kTaWaves * PPW;
  topk_row<kTaThreads, KPT, kTopkSeg, TAIL>(v, n, k, n_sink, n_local, kept, nullptr, nullptr,
                                            sm.topk, s0, s0 + kTaWaves * PPW);
  __syncthreads();

  // This workgroup's slice of the list: publish it, then attend over it.
  for (int i = tid; i < kTaWaves * PPW && s0 + i < k; i += kTaThreads)
    sel[(int64_t)unit * k + s0 + i] = kept[i];
  int pj[PPW];
  int64_t pp[PPW];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    // unconditional table loads (an empty slot reads entry 0 of the row and
    // ignores it), so that a wave's loads go out back to back
    const int i = wid * PPW + pi;
    const int j = s0 + i < k ? kept[i] : -1;
    const bool in_row = j >= 0 && j < n;
    const int64_t e = page_table[(int64_t)b * max_pages + (in_row ? j : 0)];
    pp[pi] = in_row ? e : -1;
    pj[pi] = (pp[pi] >= 0 && pp[pi] < num_pool_pages) ? j : -1;
  }
  // valid tokens of tile s of page pi (<= 0: absent); uniform over the wave
  auto tile_valid = [&](int pi, int s) {
    return pj[pi] >= 0 ? min(kTileRows, L - pj[pi] * S - s * kTileRows) : 0;
  };
  // The tile loads sit in one branch that depends on every page's table
  // entry, so all of them are in before the first tile load and no wait
  // separates the pages' loads.
  bool any = false;
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) any |= pj[pi] >= 0;
  uint4 kx[PPW][SUB][4], vx[PPW][SUB][4];
  if constexpr (G >= 2) {
    // a query group: both products on the matrix cores (dev_attn_mfma.h)
    if (any) {
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
        for (int s = 0; s < SUB; ++s)
          if (tile_valid(pi, s) > 0)
            mfma_load_tile(k_pool, v_pool, attn_tile_offset<SUB>(pp[pi], Hkv, g, s), lane,
                           kx[pi][s], vx[pi][s]);
    }
    MfmaAttnState st;
    mfma_attn_init(st);
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int v = tile_valid(pi, s);
        if (v > 0) mfma_attn_page<T>(st, qb, kx[pi][s], vx[pi][s], v, qscale, lane);
      }
    __syncthreads();  // the Top-K scratch becomes the attention scratch
    mfma_attn_stage_wave(st, sm.attn, wid, lane);
  } else {
    if (any) {
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
        for (int s = 0; s < SUB; ++s)
          if (tile_valid(pi, s) > 0)
            attn_load_tile(k_pool, v_pool, attn_tile_offset<SUB>(pp[pi], Hkv, g, s), r, c,
                           kx[pi][s], vx[pi][s]);
    }
    AttnState<G> st;
    attn_init(st);
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int v = tile_valid(pi, s);
        if (v > 0) attn_page<T, G>(st, qf, kx[pi][s], vx[pi][s], v, r);
      }
    attn_combine_rows(st);
    __syncthreads();  // the Top-K scratch becomes the attention scratch
    attn_stage_wave(st, sm.attn, wid, r, c);
  }
  __syncthreads();

  const int Hq = Hkv * G;
  for (int idx = tid; idx < G * kHeadDim; idx += kTaThreads) {
    const int h = idx / kHeadDim, ch = idx - h * kHeadDim;
    float M, den, num;
    attn_wg_partial(sm.attn, h, ch, M, den, num);
    const int64_t qh = (int64_t)b * Hq + g * G + h;
    if (nsplit == 1) {
      out[qh * kHeadDim + ch] = den > 0.f ? num / den : 0.f;
    } else {
      const int64_t slot = qh * nsplit + split;
      ws_o[slot * kHeadDim + ch] = num;
      if (ch == 0) {
        ws_ml[slot * 2] = M;
        ws_ml[slot * 2 + 1] = den;
      }
    }
  }
}

template <DType T, int G, int KPT, int PPW, int SUB, int TAIL>
void launch_t(const quest_paged_kv& kv, const void* q, const void* k_pool,
              const void* v_pool, const int32_t* page_table,
              const int32_t* seq_lens, const float* scores, int k, int n_sink,
              int n_local, float qscale, int32_t* sel, float* out, float* ws_o,
              float* ws_ml, int nsplit, hipStream_t stream) {
  dim3 grid((unsigned)nsplit, (unsigned)(kv.batch * kv.num_kv_heads));
  topk_attn_kernel<T, G, KPT, PPW, SUB, TAIL><<<grid, kTaThreads, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
      static_cast<const uint16_t*>(v_pool), page_table, seq_lens, scores, k,
      n_sink, n_local, kv.num_kv_heads, kv.max_pages_per_seq, kv.num_pool_pages, qscale, sel, out,
      ws_o, ws_ml);
}

template <DType T, int KPT, int SUB, int TAIL = 0>
void dispatch_g(int G, int ppw, const quest_paged_kv& kv, const void* q,
                const void* k_pool, const void* v_pool, const int32_t* page_table,
                const int32_t* seq_lens, const float* scores, int k, int n_sink,
                int n_local, float qscale, int32_t* sel, float* out, float* ws_o,
                float* ws_ml, int nsplit, hipStream_t s) {
#define QUEST_TA(GG, PP)                                                         \
  launch_t<T, GG, KPT, PP, SUB, TAIL>(kv, q, k_pool, v_pool, page_table, seq_lens, scores, \
                           k, n_sink, n_local, qscale, sel, out, ws_o, ws_ml,    \
                           nsplit, s)
  // ppw never exceeds the plan's limit for SUB: only those variants are built
  auto by_ppw = [&](auto gg) {
    constexpr int GG = decltype(gg)::value;
    if constexpr (SUB == 1) {
      if (ppw == 4) { QUEST_TA(GG, 4); return; }
    }
    if (ppw == 2) QUEST_TA(GG, 2);
    else QUEST_TA(GG, 1);
  };
  if (G == 1) by_ppw(std::integral_constant<int, 1>{});
  else if (G == 2) by_ppw(std::integral_constant<int, 2>{});
  else if (G == 4) by_ppw(std::integral_constant<int, 4>{});
  else by_ppw(std::integral_constant<int, 8>{});
#undef QUEST_TA
}

}  // namespace

// Scratch of quest_topk_sparse_decode_attn_noalloc: room for the split
// partials of one call, a file-scope device array (each GPU that loads the
// library holds its own copy until the process ends).  Host code must not
// pass this name to a kernel -- on the host it is only a stand-in -- but the
// device address that hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // per GPU, set once
std::mutex g_scratch_mu;

// The current GPU's address of `scratch`, looked up on the first call on
// that GPU (with the GPU current) and kept.
hipError_t scratch_address(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return hipSuccess;
}

// The 8-wave plan, and where its partials live in the caller's workspace.
struct TaLayout {
  AttnPlan pl;
  float* ws_o;
  float* ws_ml;
};

TaLayout ta_layout(const quest_paged_kv& kv, int k_pages, void* workspace) {
  TaLayout t;
  t.pl = attention_plan(kv, k_pages, kTaWaves);
  // the caller's workspace (attention_workspace_bytes, checked by every
  // entry point) holds the partials of this plan
  const size_t slots = (size_t)kv.batch * kv.num_q_heads * t.pl.nsplit;
  t.ws_o = static_cast<float*>(workspace);
  t.ws_ml = t.ws_o ? t.ws_o + attention_ml_offset(slots) : nullptr;
  return t;
}

}  // namespace

hipError_t launch_topk_attention_noalloc(const quest_paged_kv& kv, const void* q,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* page_table,
                                         const int32_t* seq_lens, const float* scores,
                                         int k_pages, int n_sink, int n_local,
                                         float sm_scale, int32_t* sel, float* out,
                                         hipStream_t stream) {
  if (attention_workspace_bytes(kv, k_pages) > kNoAllocScratchBytes)
    return hipErrorInvalidValue;  // the caller checks first
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_topk_attention(kv, q, k_pool, v_pool, page_table, seq_lens, scores,
                               k_pages, n_sink, n_local, sm_scale, sel, out, ws,
                               stream, true);
}

hipError_t launch_topk_attention_merge(const quest_paged_kv& kv, int k_pages,
                                       void* workspace, float* out,
                                       hipStream_t stream) {
  const TaLayout t = ta_layout(kv, k_pages, workspace);
  if (t.pl.nsplit > 1) launch_merge(kv, t.ws_o, t.ws_ml, t.pl.nsplit, out, stream);
  return hipGetLastError();
}

hipError_t launch_topk_attention(const quest_paged_kv& kv, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* page_table,
                                 const int32_t* seq_lens, const float* scores,
                                 int k_pages, int n_sink, int n_local,
                                 float sm_scale, int32_t* sel, float* out,
                                 void* workspace, hipStream_t stream, bool merge) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const TaLayout t = ta_layout(kv, k_pages, workspace);
  const AttnPlan pl = t.pl;
  float* ws_o = t.ws_o;
  float* ws_ml = t.ws_ml;
  const float qscale = sm_scale * kLog2e;
  const int mp = kv.max_pages_per_seq;
#define QUEST_TA_D(TT, KK, SS, TL)                                                   \
  dispatch_g<TT, KK, SS, TL>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens, \
                             scores, k_pages, n_sink, n_local, qscale, sel, out,     \
                             ws_o, ws_ml, pl.nsplit, stream)
  const bool s32 = kv.page_size == 32;
  // scores per thread: the fewest that cover the row (fewer VGPRs, a shorter
  // load and selection): 4, 4 + a tail of 1 (rows of up to 2560 pages: the
  // 32K contexts that have grown a few pages), 8 or 16
  auto by_len = [&](auto tt) {
    constexpr DType TT = decltype(tt)::value;
    if (mp <= 2048) { if (s32) QUEST_TA_D(TT, 4, 2, 0); else QUEST_TA_D(TT, 4, 1, 0); }
    else if (mp <= 2560) { if (s32) QUEST_TA_D(TT, 5, 2, 1); else QUEST_TA_D(TT, 5, 1, 1); }
    else if (mp <= 4096) { if (s32) QUEST_TA_D(TT, 8, 2, 0); else QUEST_TA_D(TT, 8, 1, 0); }
    else { if (s32) QUEST_TA_D(TT, 16, 2, 0); else QUEST_TA_D(TT, 16, 1, 0); }
  };
  if (kv.dtype == QUEST_F16) by_len(std::integral_constant<DType, DType::F16>{});
  else by_len(std::integral_constant<DType, DType::BF16>{});
#undef QUEST_TA_D
  if (merge && pl.nsplit > 1) launch_merge(kv, ws_o, ws_ml, pl.nsplit, out, stream);
  return hipGetLastError();
}

}  // namespace quest
