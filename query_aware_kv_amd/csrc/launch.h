// Host-side launchers of the Quest kernels (one per .hip file).  Each
// enqueues on `stream` and returns the launch status; arguments have been
// validated by the C ABI layer (api.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"
#include "quest.h"

namespace quest {

hipError_t launch_meta_rebuild(const quest_paged_kv& kv, const void* k_pool,
                               void* kmin, void* kmax,
                               const int32_t* page_table,
                               const int32_t* seq_lens,
                               const int32_t* first_token, hipStream_t stream);

hipError_t launch_meta_append(const quest_paged_kv& kv, void* k_pool,
                              void* v_pool, void* kmin, void* kmax,
                              const int32_t* page_table,
                              const int32_t* seq_lens, const void* k_new,
                              const void* v_new, hipStream_t stream);

// True when an estimate kernel exists for this group size.
bool estimate_supported(int group);
// per_head: one score row per query head ([B][Hq][max_pages]) instead of
// one per kv-head holding the group's sum.  k_new non-null: append token
// L_b - 1 first (k_new / v_new into k_pool / v_pool and its page's box; the
// boxes are then written, so kmin / kmax must be writable).
hipError_t launch_estimate(const quest_paged_kv& kv, const void* q,
                           const void* kmin, const void* kmax,
                           const int32_t* page_table, const int32_t* seq_lens,
                           float* scores, bool per_head, hipStream_t stream,
                           void* k_pool = nullptr, void* v_pool = nullptr,
                           const void* k_new = nullptr, const void* v_new = nullptr);

// union.hip: per (request, kv-head), the ascending union of the G query
// heads' k-entry lists, -1 padded to G*k; max_pages <= kTopkMaxPages.
hipError_t launch_union(const quest_paged_kv& kv, const int32_t* sel_heads,
                        int k_pages, int32_t* sel_union, hipStream_t stream);

// Largest max_pages_per_seq the Top-K kernel handles.
constexpr int kTopkMaxPages = 32768;
// n_sink / n_local: forced pages (0, 0 = plain Top-K); the caller checks
// n_sink + n_local <= k_pages.
hipError_t launch_topk(const quest_paged_kv& kv, const float* scores,
                       const int32_t* seq_lens, int k_pages, int n_sink,
                       int n_local, int32_t* sel, hipStream_t stream);

// Attention (sparse when sel != nullptr, else dense over all pages).
struct AttnPlan {
  int ppw;     // pages per wave
  int nsplit;  // workgroups (splits) per (request, kv-head) row
};
// waves: per workgroup (attn_split_kernel: 4; topk_attn_kernel: 8)
AttnPlan attention_plan(const quest_paged_kv& kv, int list_len, int waves = 4);
size_t attention_ml_offset(size_t slots);  // in floats, into the workspace
void launch_merge(const quest_paged_kv& kv, const float* ws_o,
                  const float* ws_ml, int nsplit, float* out,
                  hipStream_t stream);
bool attention_supported(int group);
size_t attention_workspace_bytes(const quest_paged_kv& kv, int list_len);
// Append mode of the dense attention (quest_append_decode_attn): where the
// step's token goes and the boxes it widens (null pointers otherwise).
struct AttnAppend {
  uint16_t* k_pool;
  uint16_t* v_pool;
  uint16_t* kmin;
  uint16_t* kmax;
  const uint16_t* k_new;  // [B][Hkv][128]
  const uint16_t* v_new;
};
hipError_t launch_attention(const quest_paged_kv& kv, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const int32_t* sel, int list_len, float sm_scale,
                            float* out, void* workspace, hipStream_t stream,
                            const AttnAppend* append = nullptr);
// Union mode (quest_union_sparse_decode_attn): each attention workgroup
// builds its row's union of the group's per-head lists (sel_heads
// [B][Hq][k_pages]) in LDS, walks its range of it as the sparse plan for
// G * k_pages entries gives, and writes that range to sel_union
// [B][Hkv][G * k_pages].  G * k_pages <= kUnionListMax, max_pages <=
// kTopkMaxPages.
constexpr int kUnionListMax = 4096;
hipError_t launch_union_attention(const quest_paged_kv& kv, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  const int32_t* sel_heads, int k_pages, float sm_scale,
                                  int32_t* sel_union, float* out, void* workspace,
                                  hipStream_t stream);

// Top-K + sparse attention in one launch (each workgroup selects its row).
constexpr int kTopkAttnMaxPages = 8192;
// probe.hip: streaming read of `bytes` (a multiple of 16) at `buf`.
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink,
                             hipStream_t stream);

// merge = false: leave the split partials in the workspace (out is written
// only when the plan has a single split); launch_topk_attention_merge then
// combines them.
hipError_t launch_topk_attention(const quest_paged_kv& kv, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* page_table,
                                 const int32_t* seq_lens, const float* scores,
                                 int k_pages, int n_sink, int n_local,
                                 float sm_scale, int32_t* sel, float* out,
                                 void* workspace, hipStream_t stream,
                                 bool merge = true);
hipError_t launch_topk_attention_merge(const quest_paged_kv& kv, int k_pages,
                                       void* workspace, float* out,
                                       hipStream_t stream);
// The same launches with the partials in the library's per-GPU scratch
// array (topk_attn.hip) instead of a caller workspace: no allocation.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
hipError_t launch_topk_attention_noalloc(const quest_paged_kv& kv, const void* q,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* page_table,
                                         const int32_t* seq_lens, const float* scores,
                                         int k_pages, int n_sink, int n_local,
                                         float sm_scale, int32_t* sel, float* out,
                                         hipStream_t stream);

// Fused step (estimate -> Top-K -> attention in one launch).
constexpr int kStepMaxPages = 8192;
size_t step_workspace_bytes(const quest_paged_kv& kv, int k_pages);
hipError_t launch_step(const quest_paged_kv& kv, const void* q,
                       const void* k_pool, const void* v_pool,
                       const void* kmin, const void* kmax,
                       const int32_t* page_table, const int32_t* seq_lens,
                       int k_pages, float sm_scale, float* scores,
                       int32_t* sel, float* out, void* workspace,
                       hipStream_t stream);

}  // namespace quest
