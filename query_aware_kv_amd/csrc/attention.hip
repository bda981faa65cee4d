// quest_sparse_decode_attn / quest_decode_attn: split-K flash decoding over
// page-table-indirected pages (the arithmetic lives in dev_attn.h).
//
// Workgroup = (split, request b, kv-head g), 4 waves; each wave owns PPW
// consecutive entries of the page list -- sel_pages[b][g][..] (entries -1
// skipped) or 0..n_b-1 -- and issues all of their K and V loads before any
// arithmetic (PPW * 8 KiB in flight per wave).  The four waves meet in LDS;
// with one split per row the workgroup writes the output directly, otherwise
// a partial (o[128], M, den) per query head, which the merge kernel combines.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dev_attn.h"
#include "dev_attn_mfma.h"
#include "launch.h"

namespace quest {
namespace {

// One 32-bit word (two 16-bit values) of a box widened in place by the
// token's word x: lo = min(x, lo, hi), hi = max(x, lo, hi) per value in the
// ord16 order, as folding the three with fold8 gives, with a few registers
// at a time.
__device__ __forceinline__ void widen_word(uint32_t x, uint32_t& lo, uint32_t& hi) {
  uint32_t nlo = 0, nhi = 0;
#pragma unroll
  for (int sh = 0; sh < 32; sh += 16) {
    const int32_t a = ord16(x >> sh), b = ord16(lo >> sh), c = ord16(hi >> sh);
    nlo |= unord16(min(a, min(b, c))) << sh;
    nhi |= unord16(max(a, max(b, c))) << sh;
  }
  lo = nlo;
  hi = nhi;
}

// UNION's LDS: a bitmap over the row's pages and the row's union list.
struct UnionSmem {
  uint32_t bm[kTopkMaxPages / 32];
  uint32_t wsum[kAttnWaves];
  int32_t list[kUnionListMax];
};

// The pools' pointer type: restrict-qualified unless the append mode also
// writes the pools through ap.
template <bool APPEND>
using PoolPtr = std::conditional_t<APPEND, const uint16_t*, const uint16_t* __restrict__>;

// APPEND (dense only, quest_append_decode_attn): also append token L_b - 1
// (ap.k_new / ap.v_new) to its page and widen that page's box, as
// quest_update_page_meta's append mode does.  The wave that folds that page
// loads the token with the page's tiles and puts it into the registers of
// its slot before the fold (the slot's pool bytes are not used); after its
// loop it writes the token into the pool and the widened box.  No other
// workgroup reads that page, and nothing of the append is held in registers
// across the loop, so the kernel keeps the plain instance's occupancy.
//
// UNION (sparse only, quest_union_sparse_decode_attn): `sel` holds the
// group's per-query-head lists ([b][g*G .. g*G+G-1][k], list_len = G*k
// entries from unit * list_len), and the list the workgroup walks is their
// union, built in LDS by every workgroup of the row as quest_union_pages
// builds it: the listed pages in [0, max_pages) set bits of a bitmap, the
// set bits are written out in ascending order, then -1 up to list_len.
// Each workgroup also writes its range of that list to union_out.
template <DType T, int G, int PPW, int SUB, bool APPEND = false, bool UNION = false>
__global__ void __launch_bounds__(256)
attn_split_kernel(const uint16_t* __restrict__ q,
                  PoolPtr<APPEND> k_pool,
                  PoolPtr<APPEND> v_pool,
                  const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ sel, int list_len, int Hkv,
                  int max_pages, int num_pool_pages, float qscale,
                  float* __restrict__ out, float* __restrict__ ws_o,
                  float* __restrict__ ws_ml, AttnAppend ap,
                  int32_t* __restrict__ union_out) {
  __shared__ AttnSmem<G> sm;
  __shared__ std::conditional_t<UNION, UnionSmem, int> usm;
  const int unit = blockIdx.y;  // b * Hkv + g
  const int b = unit / Hkv, g = unit - (unit / Hkv) * Hkv;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c = lane & 15, r = lane >> 4;

  // The workgroup's entries: a balanced contiguous range of the list --
  // sel_pages[b][g][..] (entries -1 skipped) or 0..max_pages-1 -- walked in
  // chunks of kAttnWaves * PPW entries, wave w taking PPW consecutive ones
  // of each chunk.  The sparse plan gives every workgroup one chunk; the
  // dense plan sizes the ranges so that the grid fits the GPU in one round.
  const int64_t lo = (int64_t)split * list_len / nsplit;
  const int64_t hi = (int64_t)(split + 1) * list_len / nsplit;
  const int L = seq_lens[b];
  constexpr int S = SUB * kTileRows;
  // APPEND: jl = the appended token's logical page when this wave folds
  // it (else -1), tl = its slot, pa = its pool page once a chunk has
  // found it valid; k_tok / v_tok = the token's K and V rows
  int jl = -1, tl = 0, pa = -1;
  const uint16_t* k_tok = nullptr;
  const uint16_t* v_tok = nullptr;
  if constexpr (APPEND) {
    const int pos = L - 1, j = pos >= 0 ? pos / S : -1;
    if (j >= 0 && j < max_pages && j >= lo && j < hi &&
        (int)((j - lo) % (kAttnWaves * PPW)) / PPW == wid) {
      jl = j;
      tl = pos - j * S;
    }
    // the same in every lane of the wave: scalar registers
    jl = __builtin_amdgcn_readfirstlane(jl);
    tl = __builtin_amdgcn_readfirstlane(tl);
    k_tok = ap.k_new + ((int64_t)b * Hkv + g) * kHeadDim;
    v_tok = ap.v_new + ((int64_t)b * Hkv + g) * kHeadDim;
  }
  // q: packed words of one head (VALU path), the MFMA operand for a group
  AttnQ<G> qf;
  uint4 qb[4];
  if constexpr (G >= 2)
    mfma_load_q<G>(q, (int64_t)unit * G, lane, qb);
  else
    attn_load_q<T, G>(q, (int64_t)unit * G, c, qscale, qf);
  MfmaAttnState mst;
  AttnState<G> vst;
  if constexpr (G >= 2) mfma_attn_init(mst);
  else attn_init(vst);
  if constexpr (UNION) {
    // The entries go out 4 per thread at a time, unconditionally from
    // clamped indices (the first 4 before the bitmap is cleared), so that
    // each group costs one round trip.
    const int32_t* src = sel + (int64_t)unit * list_len;
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = src[min(u * 256 + tid, list_len - 1)];
    const int words = (max_pages + 31) >> 5;
    for (int w = tid; w < words; w += 256) usm.bm[w] = 0u;
    __syncthreads();
    for (int base = 0; base < list_len; base += 4 * 256) {
      if (base > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = src[min(base + u * 256 + tid, list_len - 1)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * 256 + tid, p = e[u];
        if (i < list_len && p >= 0 && p < max_pages) atomicOr(&usm.bm[p >> 5], 1u << (p & 31));
      }
    }
    __syncthreads();
    // thread t owns bitmap words [t * wpt, (t + 1) * wpt); one block scan of
    // their bit counts gives each thread the list position of its first page
    const int wpt = (words + 255) >> 8, w0 = tid * wpt;
    uint32_t cnt = 0;
    for (int w = w0; w < w0 + wpt && w < words; ++w) cnt += __popc(usm.bm[w]);
    const uint32_t incl = wave_scan_incl(cnt);
    if (lane == kWave - 1) usm.wsum[wid] = incl;
    __syncthreads();
    uint32_t off = incl - cnt, total = 0;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      if (w < wid) off += usm.wsum[w];
      total += usm.wsum[w];
    }
    for (int w = w0; w < w0 + wpt && w < words; ++w) {
      uint32_t bits = usm.bm[w];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        usm.list[off++] = w * 32 + bit;
      }
    }
    for (int i = (int)total + tid; i < list_len; i += 256) usm.list[i] = -1;
    __syncthreads();
    for (int64_t i = lo + tid; i < hi; i += 256)
      union_out[(int64_t)unit * list_len + i] = usm.list[i];
  }
  for (int64_t c0 = lo; c0 < hi; c0 += kAttnWaves * PPW) {
    // List entries, then their table entries: neither waits for the length
    // (both are in bounds on their own); the length only masks afterwards.
    // The loads are unconditional, from indices clamped into the row (slots
    // past the end read a valid entry and discard it), so each group goes
    // out back to back with one wait.
    const int64_t i0 = c0 + wid * PPW;
    int jr[PPW];
    int64_t pp[PPW];
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
      const int64_t i = i0 + pi;
      if constexpr (UNION) {
        jr[pi] = i < hi ? usm.list[min(i, (int64_t)list_len - 1)] : -1;
      } else if (sel) {
        const int e = sel[(int64_t)unit * list_len + min(i, (int64_t)list_len - 1)];
        jr[pi] = i < hi ? e : -1;
      } else {
        jr[pi] = i < hi ? (int)i : -1;
      }
    }
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi) {
      const bool in_row = jr[pi] >= 0 && jr[pi] < max_pages;
      const int64_t e = page_table[(int64_t)b * max_pages + (in_row ? jr[pi] : 0)];
      pp[pi] = in_row ? e : -1;
    }
    const int n = pages_of(L, S, max_pages);
    int pj[PPW];
#pragma unroll
    for (int pi = 0; pi < PPW; ++pi)
      pj[pi] = (jr[pi] >= 0 && jr[pi] < n && pp[pi] >= 0 && pp[pi] < num_pool_pages)
                   ? jr[pi] : -1;
    // valid tokens of tile s of page pi (<= 0: absent); uniform over the wave
    auto tile_valid = [&](int pi, int s) {
      return pj[pi] >= 0 ? min(kTileRows, L - pj[pi] * S - s * kTileRows) : 0;
    };
    // APPEND: in the chunk that holds page jl, the token in the tiles'
    // layout (channels 8c of lane c; a group's MFMA K tile: channels
    // 32 s + 8 (lane / 16)), loaded with the tiles and put into the tile
    // registers of its slot before the fold (the pool's slot is not used)
    bool has = false;
    uint4 tk[4], tv = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) tk[s2] = tv;
    if constexpr (APPEND) {
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi)
        if (jl >= 0 && pj[pi] == jl) {
          has = true;
          pa = __builtin_amdgcn_readfirstlane((int)pp[pi]);  // a pool page: < num_pool_pages
        }
      if (has) {
        tv = *reinterpret_cast<const uint4*>(v_tok + c * 8);
        if constexpr (G >= 2) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
            tk[s2] = *reinterpret_cast<const uint4*>(k_tok + 32 * s2 + 8 * (lane >> 4));
        } else {
          tk[0] = *reinterpret_cast<const uint4*>(k_tok + c * 8);
        }
      }
    }
    // the tile that holds slot tl gets the token (row t in the loaders'
    // layouts: dev_attn.h, dev_attn_mfma.h)
    auto put_token = [&](uint4 (&kt)[4], uint4 (&vt)[4]) {
      const int t = tl % kTileRows;
      if constexpr (G >= 2) {
        const int jj = lane & 15;
        if ((jj & 3) * 4 + (jj >> 2) == t) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) kt[s2] = tk[s2];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e == t / 4 && (lane >> 4) == t % 4) vt[e] = tv;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (i == t / 4 && r == t % 4) {
            kt[i] = tk[0];
            vt[i] = tv;
          }
      }
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
      if constexpr (APPEND) {
        if (has) {
#pragma unroll
          for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
            for (int s = 0; s < SUB; ++s)
              if (pj[pi] == jl && s == tl / kTileRows) put_token(kx[pi][s], vx[pi][s]);
        }
      }
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          const int v = tile_valid(pi, s);
          if (v > 0) mfma_attn_page<T>(mst, qb, kx[pi][s], vx[pi][s], v, qscale, lane);
        }
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
      if constexpr (APPEND) {
        if (has) {
#pragma unroll
          for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
            for (int s = 0; s < SUB; ++s)
              if (pj[pi] == jl && s == tl / kTileRows) put_token(kx[pi][s], vx[pi][s]);
        }
      }
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
          const int v = tile_valid(pi, s);
          if (v > 0) attn_page<T, G>(vst, qf, kx[pi][s], vx[pi][s], v, r);
        }
    }
  }
  // APPEND: the token and the page's old box, loaded here (no tile is live
  // any more) and stored at the end
  uint4 kn = make_uint4(0, 0, 0, 0), vn = kn, bmin = kn, bmax = kn;
  if constexpr (APPEND) {
    if (pa >= 0 && lane < 16) {
      kn = *reinterpret_cast<const uint4*>(k_tok + lane * 8);
      vn = *reinterpret_cast<const uint4*>(v_tok + lane * 8);
      if (tl > 0) {
        const int64_t m = ((int64_t)pa * Hkv + g) * kHeadDim + lane * 8;
        bmin = *reinterpret_cast<const uint4*>(ap.kmin + m);
        bmax = *reinterpret_cast<const uint4*>(ap.kmax + m);
      }
    }
  }
  if constexpr (G >= 2) {
    mfma_attn_stage_wave(mst, sm, wid, lane);
  } else {
    attn_combine_rows(vst);
    attn_stage_wave(vst, sm, wid, r, c);
  }
  __syncthreads();

  const int Hq = Hkv * G;
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int h = idx / kHeadDim, ch = idx - h * kHeadDim;
    float M, den, num;
    attn_wg_partial(sm, h, ch, M, den, num);
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
  if constexpr (APPEND) {
    if (pa >= 0 && lane < 16) {
      const int64_t row = (((int64_t)pa * Hkv + g) * S + tl) * kHeadDim + lane * 8;
      *reinterpret_cast<uint4*>(ap.k_pool + row) = kn;
      *reinterpret_cast<uint4*>(ap.v_pool + row) = vn;
      if (tl == 0) {  // slot 0 starts the box
        bmin = kn;
        bmax = kn;
      } else {
        widen_word(kn.x, bmin.x, bmax.x);
        widen_word(kn.y, bmin.y, bmax.y);
        widen_word(kn.z, bmin.z, bmax.z);
        widen_word(kn.w, bmin.w, bmax.w);
      }
      const int64_t m = ((int64_t)pa * Hkv + g) * kHeadDim + lane * 8;
      *reinterpret_cast<uint4*>(ap.kmin + m) = bmin;
      *reinterpret_cast<uint4*>(ap.kmax + m) = bmax;
    }
  }
}

// One workgroup per (request, query head): combine its splits.  A separate
// launch: the kernel boundary publishes every split's partials, which is far
// cheaper here than per-workgroup L2 write-backs for an in-kernel hand-off.
__global__ void __launch_bounds__(256)
attn_merge_kernel(const float* __restrict__ ws_o,
                  const float* __restrict__ ws_ml, int nsplit,
                  float* __restrict__ out) {
  __shared__ MergeSmem sm;
  const int64_t qh = blockIdx.x;
  merge_splits(ws_o + qh * nsplit * kHeadDim, ws_ml + qh * nsplit * 2, nsplit,
               out + qh * kHeadDim, sm);
}

// Many splits (the dense plan's): 8 groups of 128 threads, group u folding
// splits u, u + 8, ... of every channel, 16 per memory round trip (so up to
// 128 splits take one), then the groups meet in LDS.
constexpr int kMergeWideMin = 32;
constexpr int kMergeGroups = 8;
constexpr int kMergeWideThreads = kMergeGroups * kHeadDim;

__global__ void __launch_bounds__(kMergeWideThreads)
attn_merge_wide_kernel(const float* __restrict__ ws_o,
                       const float* __restrict__ ws_ml, int nsplit,
                       float* __restrict__ out) {
  __shared__ float sm_m[kMergeGroups][kHeadDim], sm_num[kMergeGroups][kHeadDim],
      sm_den[kMergeGroups][kHeadDim];
  const int64_t qh = blockIdx.x;
  const int ch = threadIdx.x & (kHeadDim - 1), grp = threadIdx.x / kHeadDim;
  float mr = -INFINITY, num = 0.f, den = 0.f;
  merge_strided<16>(ws_o + qh * nsplit * kHeadDim, ws_ml + qh * nsplit * 2, nsplit, grp,
                    kMergeGroups, ch, mr, num, den);
  sm_m[grp][ch] = mr;
  sm_num[grp][ch] = num;
  sm_den[grp][ch] = den;
  __syncthreads();
  if (grp == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kMergeGroups; ++u) M = fmaxf(M, sm_m[u][ch]);
    float d = 0.f, nm = 0.f;
#pragma unroll
    for (int u = 0; u < kMergeGroups; ++u) {
      const float w = exp2_or_zero(sm_m[u][ch], M);
      d += sm_den[u][ch] * w;
      nm += sm_num[u][ch] * w;
    }
    out[qh * kHeadDim + ch] = d > 0.f ? nm / d : 0.f;
  }
}

// Pages per wave the registers allow: at most 4 16-token tiles per wave,
// for every group size (a group keeps its q as one 16-VGPR MFMA operand and
// its output in 32 accumulators, whatever G is).
int max_ppw(int sub) {
  constexpr int kTiles = 4;
  return kTiles / sub > 0 ? kTiles / sub : 1;
}

using Plan = AttnPlan;

}  // namespace

namespace {
// workgroups of the attention instance with `ppw` pages per wave (append
// mode or not) that the current GPU holds at once (defined below)
int64_t dense_resident(const quest_paged_kv& kv, int ppw, bool append = false);
}  // namespace

// Pages per wave: as many as the registers allow while the grid keeps at
// least ~4096 waves (16 per CU) to spread the loads over all 256 CUs -- or,
// for kernels of which fewer workgroups fit the GPU at once (query groups:
// 2 per CU at 2 pages per wave), at least as many workgroups as fit.  A grid
// between one and two resident rounds is cut to one round of balanced
// ranges instead of leaving a partial second round (a GQA layer's union
// lists: 17.4 -> 15.5 us, 512 workgroups of 2 pages per wave where there
// were 1024 of one).  The 8-wave Top-K + attention workgroups repeat the
// row's selection each, so fewer, fuller ones pay there: at least 256 of
// them (2048 waves), with at most 2 pages per wave (4 made the kernel slower
// through its registers).  Measured on the 32-head layers: 8 splits of 2
// pages per wave beat 16 of one at budgets up to 2048 tokens.  Query
// groups (G >= 2) take a candidate once the grid holds half the resident
// count, which for their 2- and 4-page instances (2 workgroups per CU) is
// one workgroup per CU: the union lists of a 32/8-head layer (8 rows of 512
// entries) then run 32 splits of 4 pages per wave, whose merge is the
// plain one, instead of 64 of 2 (union call 16.5 -> 15.5 us).
// quest_workspace_size covers the 4-wave and the 8-wave plan of a list (and,
// for whole rows, the dense plans, plain and append).
AttnPlan attention_plan(const quest_paged_kv& kv, int list_len, int waves) {
  const int64_t units = (int64_t)kv.batch * kv.num_kv_heads;
  const bool topk_wg = waves == 8;
  const int64_t min_wgs = topk_wg ? 256 : 4096 / waves;
  const int cap = topk_wg ? 2 : max_ppw(kv.page_size / kTileRows);
  int ppw = 1;
  for (int cand = min(cap, max_ppw(kv.page_size / kTileRows)); cand > 1; cand /= 2) {
    const int64_t ns = (list_len + waves * cand - 1) / (waves * cand);
    int64_t need = min_wgs;
    if (!topk_wg) {
      const int64_t resident = dense_resident(kv, cand);
      need = std::min<int64_t>(min_wgs, kv.num_q_heads > kv.num_kv_heads ? resident / 2
                                                                         : resident);
    }
    if (units * ns >= need) { ppw = cand; break; }
  }
  int nsplit = (list_len + waves * ppw - 1) / (waves * ppw);
  if (!topk_wg) {
    const int64_t res = dense_resident(kv, ppw);
    if (units * nsplit > res && units * nsplit < 2 * res)
      nsplit = (int)(res / units > 0 ? res / units : 1);
  }
  return {ppw, nsplit < 1 ? 1 : nsplit};
}

namespace {

// Workgroups of attn_split_kernel<T, G, PPW, SUB, APPEND> that the current GPU holds
// at once: the runtime's occupancy figure (from the kernel's registers and
// LDS) per CU times the CUs, looked up once per instance and GPU.  Without
// a GPU it falls back to one per CU of 256 CUs.
template <DType T, int G, int PPW, int SUB, bool APPEND = false>
int64_t resident_wgs() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  int n = dev >= 0 ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  int per_cu = 0, cus = 0;
  if (dev < 0 ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(attn_split_kernel<T, G, PPW, SUB, APPEND>), 256,
          0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                     hipSuccess || cus < 1)
    cus = 256;
  n = per_cu * cus;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The same for the instance a plan of `ppw` pages per wave launches (4 only
// for 16-token pages: max_ppw).
int64_t dense_resident(const quest_paged_kv& kv, int ppw, bool append) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  auto by_g = [&](auto tt, auto ss) -> int64_t {
    constexpr DType TT = decltype(tt)::value;
    constexpr int SS = decltype(ss)::value;
    auto pick = [&](auto gg) -> int64_t {
      constexpr int GG = decltype(gg)::value;
      if (append)  // the dense plan's shapes only (1 or 2 pages per wave)
        return ppw >= 2 ? resident_wgs<TT, GG, 2, SS, true>() : resident_wgs<TT, GG, 1, SS, true>();
      if constexpr (SS == 1) {
        if (ppw >= 4) return resident_wgs<TT, GG, 4, SS>();
      }
      return ppw >= 2 ? resident_wgs<TT, GG, 2, SS>() : resident_wgs<TT, GG, 1, SS>();
    };
    if (G == 1) return pick(std::integral_constant<int, 1>{});
    if (G == 2) return pick(std::integral_constant<int, 2>{});
    if (G == 4) return pick(std::integral_constant<int, 4>{});
    return pick(std::integral_constant<int, 8>{});
  };
  const bool s32 = kv.page_size == 32;
  if (kv.dtype == QUEST_F16)
    return s32 ? by_g(std::integral_constant<DType, DType::F16>{}, std::integral_constant<int, 2>{})
               : by_g(std::integral_constant<DType, DType::F16>{}, std::integral_constant<int, 1>{});
  return s32 ? by_g(std::integral_constant<DType, DType::BF16>{}, std::integral_constant<int, 2>{})
             : by_g(std::integral_constant<DType, DType::BF16>{}, std::integral_constant<int, 1>{});
}

}  // namespace

// Dense plan: the whole row split into balanced ranges, walked in chunks of
// 4 waves x PPW pages by as many workgroups as the GPU holds at once, so
// that no second round of a few workgroups runs alone at the end; rows of
// many requests get one workgroup each and no merge.  Single-head rows of
// 16-token pages take 2 pages per wave (4 workgroups per CU at their
// register use); query groups and 32-token pages take 1, which keeps more
// of them resident (3 per CU for a group over 16-token pages, 4 for a
// single head over 32-token pages, against 2 with 2 pages per wave).
// Measured on a 32/8-head GQA layer at 32K: 34.1 us against 39.2 us for
// 1024 workgroups of 2 pages per wave (two rounds), and 36.4 us when the
// group kernel is held to 128 VGPRs to fit 4 per CU.
AttnPlan dense_plan(const quest_paged_kv& kv, bool append = false) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const int ppw = (G == 1 && kv.page_size == kTileRows) ? 2 : 1;
  const int64_t units = (int64_t)kv.batch * kv.num_kv_heads;
  const int64_t chunks = (kv.max_pages_per_seq + kAttnWaves * ppw - 1) /
                         (kAttnWaves * ppw);
  int64_t ns = dense_resident(kv, ppw, append) / units;
  if (ns > chunks) ns = chunks;
  if (ns > 65535) ns = 65535;
  return {ppw, (int)(ns < 1 ? 1 : ns)};
}

// Workspace: [partial o: slots x 128 floats][partial (M, den): slots x 2],
// the second part 256-byte aligned.
size_t attention_ml_offset(size_t slots) {
  return ((slots * kHeadDim * sizeof(float) + 255) & ~(size_t)255) / sizeof(float);
}

void launch_merge(const quest_paged_kv& kv, const float* ws_o,
                  const float* ws_ml, int nsplit, float* out,
                  hipStream_t stream) {
  if (nsplit > kMergeWideMin)
    attn_merge_wide_kernel<<<kv.batch * kv.num_q_heads, kMergeWideThreads, 0, stream>>>(
        ws_o, ws_ml, nsplit, out);
  else
    attn_merge_kernel<<<kv.batch * kv.num_q_heads, 256, 0, stream>>>(ws_o, ws_ml, nsplit,
                                                                     out);
}

namespace {

template <DType T, int G, int PPW, int SUB, bool APPEND, bool UNION>
void launch_split(const quest_paged_kv& kv, const void* q, const void* k_pool,
                  const void* v_pool, const int32_t* page_table,
                  const int32_t* seq_lens, const int32_t* sel, int list_len,
                  float qscale, float* out, float* ws_o, float* ws_ml,
                  int nsplit, const AttnAppend& ap, int32_t* union_out,
                  hipStream_t stream) {
  dim3 grid((unsigned)nsplit, (unsigned)(kv.batch * kv.num_kv_heads));
  attn_split_kernel<T, G, PPW, SUB, APPEND, UNION><<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
      static_cast<const uint16_t*>(v_pool), page_table, seq_lens, sel,
      list_len, kv.num_kv_heads, kv.max_pages_per_seq, kv.num_pool_pages,
      qscale, out, ws_o, ws_ml, ap, union_out);
}

template <DType T, int SUB, bool APPEND, bool UNION>
void dispatch(int G, int ppw, const quest_paged_kv& kv, const void* q,
              const void* k_pool, const void* v_pool,
              const int32_t* page_table, const int32_t* seq_lens,
              const int32_t* sel, int list_len, float qscale, float* out,
              float* ws_o, float* ws_ml, int nsplit, const AttnAppend& ap,
              int32_t* union_out, hipStream_t stream) {
#define QUEST_SPLIT(GG, PP)                                                               \
  launch_split<T, GG, PP, SUB, APPEND, UNION>(kv, q, k_pool, v_pool, page_table, seq_lens, \
                                              sel, list_len, qscale, out, ws_o, ws_ml,     \
                                              nsplit, ap, union_out, stream)
  // ppw never exceeds max_ppw(SUB) (the append mode: the dense plan's 1 or
  // 2): only those variants are built
  auto by_ppw = [&](auto gg) {
    constexpr int GG = decltype(gg)::value;
    if constexpr (SUB == 1 && !APPEND) {
      if (ppw == 4) { QUEST_SPLIT(GG, 4); return; }
    }
    if (ppw == 2) QUEST_SPLIT(GG, 2);
    else QUEST_SPLIT(GG, 1);
  };
  if (G == 1) by_ppw(std::integral_constant<int, 1>{});
  else if (G == 2) by_ppw(std::integral_constant<int, 2>{});
  else if (G == 4) by_ppw(std::integral_constant<int, 4>{});
  else by_ppw(std::integral_constant<int, 8>{});
#undef QUEST_SPLIT
}

}  // namespace

bool attention_supported(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}

// Bytes of the partials of `nsplit` splits per row (0 for one split: the
// workgroups write the output themselves).
static size_t partial_bytes(const quest_paged_kv& kv, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t slots = (size_t)kv.batch * kv.num_q_heads * nsplit;
  return (attention_ml_offset(slots) + slots * 2) * sizeof(float);
}

// The sparse plans (4-wave attention, 8-wave Top-K + attention) for
// list_len entries; a list as long as the row (list_len >= max_pages_per_seq,
// the size quest_decode_attn and quest_append_decode_attn are asked with)
// also covers the dense plans.
size_t attention_workspace_bytes(const quest_paged_kv& kv, int list_len) {
  size_t need = partial_bytes(kv, attention_plan(kv, list_len).nsplit);
  const size_t t = partial_bytes(kv, attention_plan(kv, list_len, 8).nsplit);
  if (t > need) need = t;
  if (list_len >= kv.max_pages_per_seq) {
    const size_t d = partial_bytes(kv, dense_plan(kv).nsplit);
    if (d > need) need = d;
    const size_t a = partial_bytes(kv, dense_plan(kv, true).nsplit);  // append mode
    if (a > need) need = a;
  }
  return need;
}

namespace {

// union_out non-null: the union mode (sel holds the per-head lists).
hipError_t run_split_and_merge(const quest_paged_kv& kv, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* seq_lens,
                               const int32_t* sel, int list_len, float sm_scale,
                               float* out, void* workspace, hipStream_t stream,
                               const AttnAppend* append, int32_t* union_out) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  // the append mode is dense only, the union mode sparse only
  const bool app = append != nullptr && sel == nullptr;
  const bool uni = union_out != nullptr && sel != nullptr;
  const Plan pl = sel ? attention_plan(kv, list_len) : dense_plan(kv, app);
  const size_t slots = (size_t)kv.batch * kv.num_q_heads * pl.nsplit;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o ? ws_o + attention_ml_offset(slots) : nullptr;
  const float qscale = sm_scale * kLog2e;
  const AttnAppend ap = app ? *append : AttnAppend{nullptr, nullptr, nullptr, nullptr,
                                                   nullptr, nullptr};
#define QUEST_DISPATCH(TT, SS)                                                               \
  do {                                                                                       \
    if (app)                                                                                 \
      dispatch<TT, SS, true, false>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens,  \
                                    sel, list_len, qscale, out, ws_o, ws_ml, pl.nsplit, ap,  \
                                    nullptr, stream);                                        \
    else if (uni)                                                                            \
      dispatch<TT, SS, false, true>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens,  \
                                    sel, list_len, qscale, out, ws_o, ws_ml, pl.nsplit, ap,  \
                                    union_out, stream);                                      \
    else                                                                                     \
      dispatch<TT, SS, false, false>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens, \
                                     sel, list_len, qscale, out, ws_o, ws_ml, pl.nsplit, ap, \
                                     nullptr, stream);                                       \
  } while (0)
  const bool s32 = kv.page_size == 32;
  if (kv.dtype == QUEST_F16) {
    if (s32) QUEST_DISPATCH(DType::F16, 2);
    else QUEST_DISPATCH(DType::F16, 1);
  } else {
    if (s32) QUEST_DISPATCH(DType::BF16, 2);
    else QUEST_DISPATCH(DType::BF16, 1);
  }
#undef QUEST_DISPATCH
  if (pl.nsplit > 1) launch_merge(kv, ws_o, ws_ml, pl.nsplit, out, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const quest_paged_kv& kv, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const int32_t* sel, int list_len, float sm_scale,
                            float* out, void* workspace, hipStream_t stream,
                            const AttnAppend* append) {
  return run_split_and_merge(kv, q, k_pool, v_pool, page_table, seq_lens, sel, list_len,
                             sm_scale, out, workspace, stream, append, nullptr);
}

// The plan is the sparse plan for the G * k_pages entries of the union
// list, as for quest_sparse_decode_attn over quest_union_pages' output, so
// the two compositions give the same bits.
hipError_t launch_union_attention(const quest_paged_kv& kv, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  const int32_t* sel_heads, int k_pages, float sm_scale,
                                  int32_t* sel_union, float* out, void* workspace,
                                  hipStream_t stream) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  return run_split_and_merge(kv, q, k_pool, v_pool, page_table, seq_lens, sel_heads,
                             G * k_pages, sm_scale, out, workspace, stream, nullptr,
                             sel_union);
}

}  // namespace quest
