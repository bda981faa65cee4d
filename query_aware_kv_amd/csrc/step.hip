// quest_sparse_decode_step: estimate -> Top-K -> sparse attention of one
// decode step in ONE persistent launch.
//
// The steps are those of the separate calls ("Guide to Quest" §2 bound, §3
// Top-K, [paper summary] exact attention over the kept pages; arithmetic in
// dev_estimate.h, dev_topk.h, dev_attn.h).  What the fusion adds is the
// schedule:
//
//  * Work items come from one global ticket counter, in order: every
//    estimate item (64 pages of one (request, kv-head) row) before any
//    attention item (4*PPW kept pages of one row).  Workgroups grab tickets
//    until they run out.
//  * The workgroup that finishes a row's last estimate item (per-row counter)
//    runs that row's Top-K at once, writes the kept pages' pool ids next to
//    the selection, and raises the row's ready flag -- while other workgroups
//    are still estimating later rows.
//  * An attention item waits for its row's flag.  Because tickets are handed
//    out in order, every estimate item is held by a running workgroup before
//    any attention ticket exists, so every flag a waiter needs is raised by a
//    workgroup that is already running: the wait always ends, whatever the
//    grid size.  The wait is bounded all the same (a counter records a hit).
//  * The workgroup that finishes a row's last attention item merges the
//    row's split partials into the output.
//  * The last workgroup to leave resets the ticket counter; the per-row
//    counters and flags are reset by their last users.  The control block is
//    therefore all zero between calls (it must be zero before the first).
//
// Cross-workgroup hand-offs use device-scope release/acquire (the producer's
// stores are written back from its XCD's L2 before the counter or flag moves;
// the consumer invalidates before reading).
#include "dev_attn.h"
#include "dev_estimate.h"
#include "dev_topk.h"
#include "launch.h"

namespace quest {
namespace {

constexpr int kStepThreads = 256;
constexpr int kEstItemPages = (kStepThreads / 16) * kEstPages;  // 64
constexpr uint32_t kSpinLimit = 1u << 20;

struct StepCtrl {
  uint32_t ticket;  // next work item
  uint32_t exited;  // workgroups that left the item loop
  uint32_t stalls;  // waits that hit the spin limit (stays 0)
  uint32_t pad;
};

struct StepArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const uint16_t* kmin;
  const uint16_t* kmax;
  const int32_t* page_table;
  const int32_t* seq_lens;
  float* scores;
  int32_t* sel;
  float* out;
  StepCtrl* ctrl;
  uint32_t* est_done;   // [rows]
  uint32_t* ready;      // [rows]
  uint32_t* attn_done;  // [rows]
  int32_t* phys;        // [rows][k] pool ids of the kept pages, -1 padded
  float* ws_o;          // [rows * G][attn_items][128]
  float* ws_ml;         // [rows * G][attn_items][2]
  int Hkv, max_pages, num_pool_pages, k;
  int est_items, attn_items;  // per row
  uint32_t n_est, n_attn;     // in total
  float qscale;
};

__device__ __forceinline__ void fence_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire() {
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ uint32_t fetch_add_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int row_pages(const StepArgs& a, int b) {
  const int L = a.seq_lens[b];
  return pages_of(L, kTileRows, a.max_pages);  // 16-token pages only
}

template <int G>
union StepSmem {
  TopkSmem<kStepThreads> topk;
  AttnSmem<G> attn;
  MergeSmem merge;
};

template <DType T, int G, int KPT>
__device__ __forceinline__ void est_item(const StepArgs& a, uint32_t t, StepSmem<G>& sm,
                         uint32_t& flag) {
  const int tid = threadIdx.x;
  const int row = t / a.est_items, blk = t - row * a.est_items;
  const int b = row / a.Hkv, g = row - b * a.Hkv;
  const int n = row_pages(a, b);
  const int counted = max(1, (n + kEstItemPages - 1) / kEstItemPages);
  const int c = tid & 15;
  const int j0 = blk * kEstItemPages + (tid >> 4) * kEstPages;
  const int32_t* pt_row = a.page_table + (int64_t)b * a.max_pages;
  float* srow = a.scores + (int64_t)row * a.max_pages;
  if (j0 < a.max_pages) {
    EstQ<G> qq;
    est_load_q<G>(a.q, (int64_t)row * G, c, qq);
    int ent[kEstPages], pid[kEstPages];
    est_table(pt_row, a.max_pages, j0, ent);
    est_page_ids(ent, n, j0, a.num_pool_pages, pid);
    uint4 lo[kEstPages], hi[kEstPages];
    est_load_meta(a.kmin, a.kmax, pid, a.Hkv, g, c, lo, hi);
    float s[kEstPages];
    est_score<T, G>(qq, pid, lo, hi, s);
    est_store(srow, j0, a.max_pages, c, pid, s);
  }
  if (blk >= counted) return;  // a padding-only item: nobody waits for it
  fence_release();
  __syncthreads();
  if (tid == 0) flag = fetch_add_acq_rel(&a.est_done[row], 1u) == (uint32_t)(counted - 1);
  __syncthreads();
  if (!flag) return;
  // Last estimate item of this row: select now.
  fence_acquire();
  float v[KPT];
  int32_t ent[KPT];
  topk_load<kStepThreads, KPT>(srow, n, v);
  topk_load_table<kStepThreads, KPT>(pt_row, n, ent);
  topk_row<kStepThreads, KPT>(v, n, a.k, 0, 0, a.sel + (int64_t)row * a.k, &ent,
                              a.phys + (int64_t)row * a.k, sm.topk);
  fence_release();
  __syncthreads();
  if (tid == 0) {
    a.est_done[row] = 0;
    __hip_atomic_store(&a.ready[row], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <DType T, int G, int PPW>
__device__ __forceinline__ void attn_item(const StepArgs& a, uint32_t t, StepSmem<G>& sm,
                          uint32_t& flag) {
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c = lane & 15, r = lane >> 4;
  const int row = t / a.attn_items, split = t - row * a.attn_items;
  const int b = row / a.Hkv, g = row - b * a.Hkv;
  const int L = a.seq_lens[b];
  const int n = row_pages(a, b);
  if (tid == 0) {
    // Poll with relaxed loads (no cache invalidation per poll); the single
    // acquire fence below orders what follows after the flag.  The first
    // wait to reach the limit raises `stalls`, which ends every other wait.
    uint32_t spins = 0;
    while (__hip_atomic_load(&a.ready[row], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (++spins > kSpinLimit) {
        atomicAdd(&a.ctrl->stalls, 1u);
        break;
      }
      if ((spins & 63u) == 0u &&
          __hip_atomic_load(&a.ctrl->stalls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
        break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  fence_acquire();

  AttnQ<G> qf;
  attn_load_q<T, G>(a.q, (int64_t)row * G, c, a.qscale, qf);
  const int i0 = (split * kAttnWaves + wid) * PPW;
  int pj[PPW];
  int64_t pp[PPW];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int i = i0 + pi;
    int j = -1, p = -1;
    if (i < a.k) {
      j = a.sel[(int64_t)row * a.k + i];
      p = a.phys[(int64_t)row * a.k + i];
    }
    const bool ok = j >= 0 && j < n && p >= 0 && p < a.num_pool_pages;
    pj[pi] = ok ? j : -1;
    pp[pi] = p;
  }
  uint4 kx[PPW][4], vx[PPW][4];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi)
    if (pj[pi] >= 0)
      attn_load_tile(a.k_pool, a.v_pool, attn_tile_offset<1>(pp[pi], a.Hkv, g, 0), r, c,
                     kx[pi], vx[pi]);
  AttnState<G> st;
  attn_init(st);
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi)
    if (pj[pi] >= 0)
      attn_page<T, G>(st, qf, kx[pi], vx[pi], min(kTileRows, L - pj[pi] * kTileRows), r);
  attn_combine_rows(st);
  attn_stage_wave(st, sm.attn, wid, r, c);
  __syncthreads();

  const int Hq = a.Hkv * G;
  const int nsplit = a.attn_items;
  for (int idx = tid; idx < G * kHeadDim; idx += kStepThreads) {
    const int h = idx / kHeadDim, ch = idx - h * kHeadDim;
    float M, den, num;
    attn_wg_partial(sm.attn, h, ch, M, den, num);
    if (nsplit == 1) {
      a.out[((int64_t)b * Hq + g * G + h) * kHeadDim + ch] = den > 0.f ? num / den : 0.f;
    } else {
      const int64_t slot = ((int64_t)row * G + h) * nsplit + split;
      a.ws_o[slot * kHeadDim + ch] = num;
      if (ch == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = den;
      }
    }
  }
  if (nsplit == 1) {
    __syncthreads();
    if (tid == 0) a.ready[row] = 0;
    return;
  }
  fence_release();
  __syncthreads();
  if (tid == 0) flag = fetch_add_acq_rel(&a.attn_done[row], 1u) == (uint32_t)(nsplit - 1);
  __syncthreads();
  if (!flag) return;
  // Last attention item of this row: merge its splits.
  fence_acquire();
  for (int h = 0; h < G; ++h) {
    const int64_t first = ((int64_t)row * G + h) * nsplit;
    merge_splits(a.ws_o + first * kHeadDim, a.ws_ml + first * 2, nsplit,
                 a.out + ((int64_t)b * Hq + g * G + h) * kHeadDim, sm.merge);
    __syncthreads();
  }
  if (tid == 0) {
    a.attn_done[row] = 0;
    a.ready[row] = 0;
  }
}

template <DType T, int G, int KPT, int PPW>
__global__ void __launch_bounds__(kStepThreads)
step_kernel(StepArgs a) {
  __shared__ StepSmem<G> sm;
  __shared__ uint32_t sh_ticket, sh_flag;
  const int tid = threadIdx.x;
  const uint32_t total = a.n_est + a.n_attn;
  for (;;) {
    if (tid == 0) sh_ticket = atomicAdd(&a.ctrl->ticket, 1u);
    __syncthreads();
    const uint32_t t = sh_ticket;
    __syncthreads();
    if (t >= total) break;
    if (t < a.n_est)
      est_item<T, G, KPT>(a, t, sm, sh_flag);
    else
      attn_item<T, G, PPW>(a, t - a.n_est, sm, sh_flag);
  }
  if (tid == 0) {
    const uint32_t left = fetch_add_acq_rel(&a.ctrl->exited, 1u);
    if (left == gridDim.x - 1) {  // last one out: ready the queue for the next call
      a.ctrl->ticket = 0;
      a.ctrl->exited = 0;
      // a stalled wait of this call must not cut short the waits of the
      // next one: every wait ends at once while `stalls` is non-zero
      a.ctrl->stalls = 0;
    }
  }
}

// ------------------------------------------------------------------ host

struct StepPlan {
  int kpt, ppw, est_items, attn_items;
  size_t off_rows, off_phys, off_o, off_ml, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

StepPlan step_plan(const quest_paged_kv& kv, int k) {
  StepPlan p{};
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const int64_t rows = (int64_t)kv.batch * kv.num_kv_heads;
  p.kpt = kv.max_pages_per_seq <= 2048 ? 8 : 32;
  const int64_t items1 = rows * ((k + kAttnWaves - 1) / kAttnWaves);
  p.ppw = (G <= 4 && items1 > 4096) ? 2 : 1;
  p.est_items = (kv.max_pages_per_seq + kEstItemPages - 1) / kEstItemPages;
  p.attn_items = (k + kAttnWaves * p.ppw - 1) / (kAttnWaves * p.ppw);
  size_t off = align256(sizeof(StepCtrl));
  p.off_rows = off;
  off += align256(3 * rows * sizeof(uint32_t));
  p.off_phys = off;
  off += align256((size_t)rows * k * sizeof(int32_t));
  const size_t slots = (size_t)rows * G * p.attn_items;
  p.off_o = off;
  off += align256(slots * kHeadDim * sizeof(float));
  p.off_ml = off;
  off += align256(slots * 2 * sizeof(float));
  p.bytes = off;
  return p;
}

// Resident workgroups of one kernel on the whole device (cached per kernel).
template <DType T, int G, int KPT, int PPW>
int grid_for(uint32_t items) {
  static int per_cu = -1, cus = -1;  // one cache per kernel instantiation
  if (per_cu < 0) {
    auto kernel = step_kernel<T, G, KPT, PPW>;
    int dev = 0, nb = 0, ncu = 0;
    (void)hipGetDevice(&dev);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, kStepThreads, 0) != hipSuccess || nb < 1)
      nb = 1;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
      ncu = 1;
    cus = ncu;
    per_cu = nb;
  }
  const int64_t g = (int64_t)per_cu * cus;
  return (int)(items < (uint32_t)g ? items : g);
}

template <DType T, int G, int KPT, int PPW>
void launch_t(const StepArgs& a, hipStream_t stream) {
  const int grid = grid_for<T, G, KPT, PPW>(a.n_est + a.n_attn);
  step_kernel<T, G, KPT, PPW><<<grid, kStepThreads, 0, stream>>>(a);
}

template <DType T, int G>
void dispatch_kpt_ppw(int kpt, int ppw, const StepArgs& a, hipStream_t s) {
  if (kpt == 8) {
    if (ppw == 2 && G <= 4) launch_t<T, G, 8, (G <= 4 ? 2 : 1)>(a, s);
    else launch_t<T, G, 8, 1>(a, s);
  } else {
    if (ppw == 2 && G <= 4) launch_t<T, G, 32, (G <= 4 ? 2 : 1)>(a, s);
    else launch_t<T, G, 32, 1>(a, s);
  }
}

template <DType T>
void dispatch(int G, int kpt, int ppw, const StepArgs& a, hipStream_t s) {
  switch (G) {
    case 1: dispatch_kpt_ppw<T, 1>(kpt, ppw, a, s); break;
    case 2: dispatch_kpt_ppw<T, 2>(kpt, ppw, a, s); break;
    case 4: dispatch_kpt_ppw<T, 4>(kpt, ppw, a, s); break;
    default: dispatch_kpt_ppw<T, 8>(kpt, ppw, a, s); break;
  }
}

}  // namespace

size_t step_workspace_bytes(const quest_paged_kv& kv, int k_pages) {
  return step_plan(kv, k_pages).bytes;
}

hipError_t launch_step(const quest_paged_kv& kv, const void* q,
                       const void* k_pool, const void* v_pool,
                       const void* kmin, const void* kmax,
                       const int32_t* page_table, const int32_t* seq_lens,
                       int k_pages, float sm_scale, float* scores,
                       int32_t* sel, float* out, void* workspace,
                       hipStream_t stream) {
  const StepPlan p = step_plan(kv, k_pages);
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const int64_t rows = (int64_t)kv.batch * kv.num_kv_heads;
  char* ws = static_cast<char*>(workspace);
  StepArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.kmin = static_cast<const uint16_t*>(kmin);
  a.kmax = static_cast<const uint16_t*>(kmax);
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.scores = scores;
  a.sel = sel;
  a.out = out;
  a.ctrl = reinterpret_cast<StepCtrl*>(ws);
  a.est_done = reinterpret_cast<uint32_t*>(ws + p.off_rows);
  a.ready = a.est_done + rows;
  a.attn_done = a.ready + rows;
  a.phys = reinterpret_cast<int32_t*>(ws + p.off_phys);
  a.ws_o = reinterpret_cast<float*>(ws + p.off_o);
  a.ws_ml = reinterpret_cast<float*>(ws + p.off_ml);
  a.Hkv = kv.num_kv_heads;
  a.max_pages = kv.max_pages_per_seq;
  a.num_pool_pages = kv.num_pool_pages;
  a.k = k_pages;
  a.est_items = p.est_items;
  a.attn_items = p.attn_items;
  a.n_est = (uint32_t)(rows * p.est_items);
  a.n_attn = (uint32_t)(rows * p.attn_items);
  a.qscale = sm_scale * kLog2e;
  if (kv.dtype == QUEST_F16)
    dispatch<DType::F16>(G, p.kpt, p.ppw, a, stream);
  else
    dispatch<DType::BF16>(G, p.kpt, p.ppw, a, stream);
  return hipGetLastError();
}

}  // namespace quest
