// Split-K flash-decoding attention over page-table-indirected pages.
//
// Sparse: "Quest: Query-Aware Sparsity for Efficient Long-Context LLM
// Inference" (paper summary), Summary, and "Guide to Quest", §3: exact
// softmax attention over only the kept pages' tokens.  Dense: the attention
// equation of "The Memory Bandwidth Bottleneck of Long-Context Decoding"
// (Guide to Quest) over every page.  One kernel serves both; the page list
// is sel_pages[b][g][0..list_len) (entries -1 skipped) or 0..n_b-1.
//
// Work mapping.  Workgroup = (split, request b, kv-head g), 4 waves; each
// wave owns PPW consecutive list entries and issues all of their K and V
// loads before any arithmetic (up to PPW * 8 KiB in flight per wave).
// Within a wave, lane = 16 r + c holds channels 8c..8c+7 of token rows
// r, r+4, r+8, r+12 of each page: every load instruction reads 1 KiB
// contiguous, every byte is read by exactly one lane, and the q.k dot of a
// row is a DPP row reduction.  Each row group r keeps its own online-softmax
// state (m, l, o) over its tokens, so the loop needs no cross-row traffic;
// the four row groups, then the four waves (through LDS), then the splits
// (merge kernel) are combined with the usual rescaling.  Softmax runs in the
// exp2 domain with sm_scale * log2(e) folded into q; accumulation is float32.
// Tokens past a request's end are masked by selection, never by
// multiplication, so the unused slots may hold NaN.
#include "common.h"
#include "launch.h"

namespace quest {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;

template <DType T, int G, int PPW>
__global__ void __launch_bounds__(256)
attn_split_kernel(const uint16_t* __restrict__ q,
                  const uint16_t* __restrict__ k_pool,
                  const uint16_t* __restrict__ v_pool,
                  const int32_t* __restrict__ page_table,
                  const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ sel, int list_len, int Hkv,
                  int max_pages, int num_pool_pages, float qscale,
                  float* __restrict__ out,
                  float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  const int unit = blockIdx.y;  // b * Hkv + g
  const int b = unit / Hkv, g = unit - (unit / Hkv) * Hkv;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int c = lane & 15, r = lane >> 4;
  const int L = seq_lens[b];
  const int n = L > 0 ? min((L + kPageSize - 1) / kPageSize, max_pages) : 0;
  const int Hq = Hkv * G;

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t off = ((int64_t)unit * G + h) * kHeadDim + c * 8;
    widen8<T>(*reinterpret_cast<const uint4*>(q + off), qf[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[h][e] *= qscale;
  }

  // This wave's pages.
  const int i0 = (split * kWavesPerBlock + wid) * PPW;
  int pj[PPW];
  uint4 kx[PPW][4], vx[PPW][4];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int i = i0 + pi;
    int j = -1;
    if (sel) {
      if (i < list_len) j = sel[(int64_t)unit * list_len + i];
    } else if (i < n) {
      j = i;
    }
    if (j >= n) j = -1;
    pj[pi] = j;
  }
  int64_t pp[PPW];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    pp[pi] = pj[pi] >= 0 ? page_table[(int64_t)b * max_pages + pj[pi]] : -1;
    if (pp[pi] < 0 || pp[pi] >= num_pool_pages) pj[pi] = -1;  // not a pool page
  }
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    if (pj[pi] < 0) continue;
    const int64_t p = pp[pi];
    const int64_t tile = (p * Hkv + g) * (kPageSize * kHeadDim) + c * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kx[pi][i] = *reinterpret_cast<const uint4*>(k_pool + tile + (r + 4 * i) * kHeadDim);
      vx[pi][i] = *reinterpret_cast<const uint4*>(v_pool + tile + (r + 4 * i) * kHeadDim);
    }
  }

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }

#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    if (pj[pi] < 0) continue;
    const int v = min(kPageSize, L - pj[pi] * kPageSize);
    bool valid[4];
    float kf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      valid[i] = r + 4 * i < v;
      widen8<T>(kx[pi][i], kf[i]);
    }
    float z[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qf[h][e], kf[i][e], acc);
        z[h][i] = row16_sum(acc);
      }
    float vf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      widen8<T>(vx[pi][i], vf[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[i][e] = valid[i] ? vf[i][e] : 0.f;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = valid[i] ? fmaxf(mx, z[h][i]) : mx;
      const float alpha = exp2_or_zero(m[h], mx);
      float p[4], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = valid[i] ? exp2f(z[h][i] - mx) : 0.f;
        ps += p[i];
      }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = o[h][e] * alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(p[i], vf[i][e], acc);
        o[h][e] = acc;
      }
      m[h] = mx;
    }
  }

  // Combine the four row groups (lanes c, c+16, c+32, c+48).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = shfl_xor_f(m[h], off), lo = shfl_xor_f(l[h], off);
      const float M = fmaxf(m[h], mo);
      const float sa = exp2_or_zero(m[h], M), sb = exp2_or_zero(mo, M);
      l[h] = l[h] * sa + lo * sb;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[h][e] = o[h][e] * sa + shfl_xor_f(o[h][e], off) * sb;
      m[h] = M;
    }
  }

  // Combine the four waves.
  __shared__ float sm_o[kWavesPerBlock][G][kHeadDim];
  __shared__ float sm_m[kWavesPerBlock][G], sm_l[kWavesPerBlock][G];
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wid][h][c * 8 + e] = o[h][e];
      if (c == 0) {
        sm_m[wid][h] = m[h];
        sm_l[wid][h] = l[h];
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kHeadDim; idx += 256) {
    const int h = idx / kHeadDim, ch = idx - h * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) M = fmaxf(M, sm_m[w][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const float s = exp2_or_zero(sm_m[w][h], M);
      den += sm_l[w][h] * s;
      num += sm_o[w][h][ch] * s;
    }
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

// One workgroup per (request, query head): combine its splits.
__global__ void __launch_bounds__(128)
attn_merge_kernel(const float* __restrict__ ws_o,
                  const float* __restrict__ ws_ml, int nsplit,
                  float* __restrict__ out) {
  const int64_t qh = blockIdx.x;
  const int ch = threadIdx.x;
  const float* ml = ws_ml + qh * nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f, num = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float w = exp2_or_zero(ml[2 * s], M);
    den += ml[2 * s + 1] * w;
    num += ws_o[(qh * nsplit + s) * kHeadDim + ch] * w;
  }
  out[qh * kHeadDim + ch] = den > 0.f ? num / den : 0.f;
}

int max_ppw(int G) { return G == 1 ? 4 : G <= 4 ? 2 : 1; }

struct Plan {
  int ppw;
  int nsplit;
};

// Pages per wave: as many as the group size allows while the grid keeps at
// least ~1024 workgroups (4 per CU) to spread the loads over all 256 CUs.
Plan plan(const quest_paged_kv& kv, int list_len) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const int64_t units = (int64_t)kv.batch * kv.num_kv_heads;
  int ppw = 1;
  for (int cand = max_ppw(G); cand > 1; cand /= 2) {
    const int64_t ns = (list_len + kWavesPerBlock * cand - 1) / (kWavesPerBlock * cand);
    if (units * ns >= 1024) { ppw = cand; break; }
  }
  const int nsplit = (list_len + kWavesPerBlock * ppw - 1) / (kWavesPerBlock * ppw);
  return {ppw, nsplit < 1 ? 1 : nsplit};
}

template <DType T, int G, int PPW>
void launch_split(const quest_paged_kv& kv, const void* q, const void* k_pool,
                  const void* v_pool, const int32_t* page_table,
                  const int32_t* seq_lens, const int32_t* sel, int list_len,
                  float qscale, float* out, float* ws_o, float* ws_ml,
                  int nsplit, hipStream_t stream) {
  dim3 grid((unsigned)nsplit, (unsigned)(kv.batch * kv.num_kv_heads));
  attn_split_kernel<T, G, PPW><<<grid, 256, 0, stream>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_pool),
      static_cast<const uint16_t*>(v_pool), page_table, seq_lens, sel,
      list_len, kv.num_kv_heads, kv.max_pages_per_seq, kv.num_pool_pages,
      qscale, out, ws_o, ws_ml);
}

template <DType T>
void dispatch(int G, int ppw, const quest_paged_kv& kv, const void* q,
              const void* k_pool, const void* v_pool,
              const int32_t* page_table, const int32_t* seq_lens,
              const int32_t* sel, int list_len, float qscale, float* out,
              float* ws_o, float* ws_ml, int nsplit, hipStream_t stream) {
#define QUEST_SPLIT(GG, PP)                                                   \
  launch_split<T, GG, PP>(kv, q, k_pool, v_pool, page_table, seq_lens, sel,  \
                          list_len, qscale, out, ws_o, ws_ml, nsplit, stream)
  if (G == 1) {
    if (ppw == 4) QUEST_SPLIT(1, 4);
    else if (ppw == 2) QUEST_SPLIT(1, 2);
    else QUEST_SPLIT(1, 1);
  } else if (G == 2) {
    if (ppw == 2) QUEST_SPLIT(2, 2);
    else QUEST_SPLIT(2, 1);
  } else if (G == 4) {
    if (ppw == 2) QUEST_SPLIT(4, 2);
    else QUEST_SPLIT(4, 1);
  } else {
    QUEST_SPLIT(8, 1);
  }
#undef QUEST_SPLIT
}

}  // namespace

bool attention_supported(int group) {
  return group == 1 || group == 2 || group == 4 || group == 8;
}

size_t attention_workspace_bytes(const quest_paged_kv& kv, int list_len) {
  const Plan pl = plan(kv, list_len);
  if (pl.nsplit == 1) return 0;
  const size_t slots = (size_t)kv.batch * kv.num_q_heads * pl.nsplit;
  return slots * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attention(const quest_paged_kv& kv, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const int32_t* sel, int list_len, float sm_scale,
                            float* out, void* workspace, hipStream_t stream) {
  const int G = kv.num_q_heads / kv.num_kv_heads;
  const Plan pl = plan(kv, list_len);
  const size_t slots = (size_t)kv.batch * kv.num_q_heads * pl.nsplit;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o ? ws_o + slots * kHeadDim : nullptr;
  const float qscale = sm_scale * kLog2e;
  if (kv.dtype == QUEST_F16)
    dispatch<DType::F16>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens,
                         sel, list_len, qscale, out, ws_o, ws_ml, pl.nsplit, stream);
  else
    dispatch<DType::BF16>(G, pl.ppw, kv, q, k_pool, v_pool, page_table, seq_lens,
                          sel, list_len, qscale, out, ws_o, ws_ml, pl.nsplit, stream);
  if (pl.nsplit > 1) {
    attn_merge_kernel<<<kv.batch * kv.num_q_heads, kHeadDim, 0, stream>>>(
        ws_o, ws_ml, pl.nsplit, out);
  }
  return hipGetLastError();
}

}  // namespace quest
