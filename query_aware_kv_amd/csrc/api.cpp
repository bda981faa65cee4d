// C ABI of libquest.so: argument validation, dispatch and error reporting.
// Every entry point checks its arguments on the host, then enqueues kernels
// on the caller's stream; nothing is allocated and no state is kept.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"
#include "launch.h"
#include "quest.h"

namespace {

// The one-launch step kernel (step.hip) did not complete on gfx950 in its
// first runs, and the cause is not yet found; its entry point refuses work
// before any launch until it is.
constexpr bool kFusedStepEnabled = false;

thread_local char g_last_error[512] = "";

quest_status fail(quest_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

quest_status ok() {
  g_last_error[0] = '\0';
  return QUEST_OK;
}

quest_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(QUEST_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

#define REQUIRE_PTR(p, align_ok)                                               \
  do {                                                                         \
    if ((p) == nullptr)                                                        \
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `%s` is NULL", fn, #p);     \
    if (!(align_ok))                                                           \
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `%s` is misaligned", fn, #p); \
  } while (0)

quest_status check_kv(const quest_paged_kv* kv, const char* fn) {
  if (kv == nullptr)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `kv` is NULL", fn);
  if (kv->batch < 1 || kv->num_kv_heads < 1 || kv->num_q_heads < 1 ||
      kv->num_pool_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: batch, heads, num_pool_pages and max_pages_per_seq must "
                "be >= 1", fn);
  if (kv->num_q_heads % kv->num_kv_heads != 0)
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                fn, kv->num_q_heads, kv->num_kv_heads);
  if (kv->head_dim != quest::kHeadDim)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: head_dim %d (only 128)", fn,
                kv->head_dim);
  if (!quest::page_size_supported(kv->page_size))
    return fail(QUEST_ERR_UNSUPPORTED, "%s: page_size %d (16 or 32)", fn,
                kv->page_size);
  if (kv->dtype != QUEST_F16 && kv->dtype != QUEST_BF16)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: dtype %d", fn, kv->dtype);
  if ((int64_t)kv->batch * kv->num_q_heads > (int64_t)1 << 30 ||
      (int64_t)kv->batch * kv->num_kv_heads > 65535)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: batch x heads too large", fn);
  return QUEST_OK;
}

quest_status check_topk_counts(int32_t k_pages, int32_t n_sink, int32_t n_local,
                               const char* fn) {
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  if (n_sink < 0 || n_local < 0 || (int64_t)n_sink + n_local > k_pages)
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: need 0 <= n_sink, 0 <= n_local, n_sink + n_local <= k_pages "
                "(got %d, %d, k_pages %d)", fn, n_sink, n_local, k_pages);
  return QUEST_OK;
}

// The plain entry points forward to the _ex ones; their messages then name
// the entry point the caller used.
void retag(char* msg, const char* from, const char* to) {
  const size_t nf = strlen(from);
  if (strncmp(msg, from, nf) != 0) return;
  char tmp[sizeof(g_last_error)];
  snprintf(tmp, sizeof(tmp), "%s%s", to, msg + nf);
  snprintf(msg, sizeof(g_last_error), "%s", tmp);
}

quest_status check_group(const quest_paged_kv* kv, const char* fn) {
  const int G = kv->num_q_heads / kv->num_kv_heads;
  if (!quest::estimate_supported(G) || !quest::attention_supported(G))
    return fail(QUEST_ERR_UNSUPPORTED, "%s: group size %d (1, 2, 4 or 8)", fn, G);
  return QUEST_OK;
}

quest_status check_attention_common(const quest_paged_kv* kv, const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* page_table,
                                    const int32_t* seq_lens, float sm_scale,
                                    const float* out, const char* fn) {
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  REQUIRE_PTR(q, aligned16(q));
  REQUIRE_PTR(k_pool, aligned16(k_pool));
  REQUIRE_PTR(v_pool, aligned16(v_pool));
  REQUIRE_PTR(page_table, aligned4(page_table));
  REQUIRE_PTR(seq_lens, aligned4(seq_lens));
  REQUIRE_PTR(out, aligned4(out));
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: sm_scale is not finite", fn);
  return QUEST_OK;
}

// The attention workspace for a list of list_len entries.
quest_status check_attention_workspace(const quest_paged_kv* kv, int list_len,
                                       const void* workspace, size_t workspace_bytes,
                                       const char* fn) {
  const size_t need = quest::attention_workspace_bytes(*kv, list_len);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(QUEST_ERR_WORKSPACE_TOO_SMALL,
                  "%s: workspace needs %zu bytes, got %zu", fn, need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace))
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `workspace` is misaligned", fn);
  }
  return QUEST_OK;
}

quest_status run_attention(const quest_paged_kv* kv, const void* q,
                           const void* k_pool, const void* v_pool,
                           const int32_t* page_table, const int32_t* seq_lens,
                           const int32_t* sel, int list_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes,
                           void* stream, const char* fn,
                           const quest::AttnAppend* append = nullptr) {
  const quest_status s =
      check_attention_workspace(kv, list_len, workspace, workspace_bytes, fn);
  if (s != QUEST_OK) return s;
  return hip_status(
      quest::launch_attention(*kv, q, k_pool, v_pool, page_table, seq_lens, sel,
                              list_len, sm_scale, out, workspace,
                              static_cast<hipStream_t>(stream), append),
      fn);
}

}  // namespace

extern "C" {

QUEST_API quest_status quest_update_page_meta(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin,
    void* kmax, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* first_token, const void* k_new, const void* v_new,
    void* stream) {
  const char* fn = "quest_update_page_meta";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(k_pool, aligned16(k_pool));
  REQUIRE_PTR(kmin, aligned16(kmin));
  REQUIRE_PTR(kmax, aligned16(kmax));
  REQUIRE_PTR(page_table, aligned4(page_table));
  REQUIRE_PTR(seq_lens, aligned4(seq_lens));
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: k_new and v_new must both be set (append) or both NULL "
                "(rebuild)", fn);
  if (k_new == nullptr) {
    if (first_token != nullptr && !aligned4(first_token))
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `first_token` is misaligned", fn);
    return hip_status(quest::launch_meta_rebuild(
                          *kv, k_pool, kmin, kmax, page_table, seq_lens,
                          first_token, static_cast<hipStream_t>(stream)),
                      fn);
  }
  if (first_token != nullptr)
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: first_token must be NULL in append mode", fn);
  REQUIRE_PTR(v_pool, aligned16(v_pool));
  REQUIRE_PTR(k_new, aligned16(k_new));
  REQUIRE_PTR(v_new, aligned16(v_new));
  return hip_status(quest::launch_meta_append(*kv, k_pool, v_pool, kmin, kmax,
                                              page_table, seq_lens, k_new,
                                              v_new,
                                              static_cast<hipStream_t>(stream)),
                    fn);
}

static quest_status run_estimate(const quest_paged_kv* kv, const void* q,
                          const void* kmin, const void* kmax,
                          const int32_t* page_table, const int32_t* seq_lens,
                          float* scores, bool per_head, void* stream,
                          const char* fn) {
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  REQUIRE_PTR(q, aligned16(q));
  REQUIRE_PTR(kmin, aligned16(kmin));
  REQUIRE_PTR(kmax, aligned16(kmax));
  REQUIRE_PTR(page_table, aligned4(page_table));
  REQUIRE_PTR(seq_lens, aligned4(seq_lens));
  REQUIRE_PTR(scores, aligned4(scores));
  return hip_status(quest::launch_estimate(*kv, q, kmin, kmax, page_table,
                                           seq_lens, scores, per_head,
                                           static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_estimate(const quest_paged_kv* kv, const void* q,
                                      const void* kmin, const void* kmax,
                                      const int32_t* page_table,
                                      const int32_t* seq_lens, float* scores,
                                      void* stream) {
  return run_estimate(kv, q, kmin, kmax, page_table, seq_lens, scores, false,
                      stream, "quest_estimate");
}

QUEST_API quest_status quest_append_estimate(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin, void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, const void* k_new,
    const void* v_new, const void* q, float* scores, void* stream) {
  const char* fn = "quest_append_estimate";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  REQUIRE_PTR(k_pool, aligned16(k_pool));
  REQUIRE_PTR(v_pool, aligned16(v_pool));
  REQUIRE_PTR(k_new, aligned16(k_new));
  REQUIRE_PTR(v_new, aligned16(v_new));
  REQUIRE_PTR(q, aligned16(q));
  REQUIRE_PTR(kmin, aligned16(kmin));
  REQUIRE_PTR(kmax, aligned16(kmax));
  REQUIRE_PTR(page_table, aligned4(page_table));
  REQUIRE_PTR(seq_lens, aligned4(seq_lens));
  REQUIRE_PTR(scores, aligned4(scores));
  return hip_status(quest::launch_estimate(*kv, q, kmin, kmax, page_table, seq_lens,
                                           scores, false,
                                           static_cast<hipStream_t>(stream), k_pool,
                                           v_pool, k_new, v_new),
                    fn);
}

QUEST_API quest_status quest_estimate_heads(const quest_paged_kv* kv,
                                            const void* q, const void* kmin,
                                            const void* kmax,
                                            const int32_t* page_table,
                                            const int32_t* seq_lens,
                                            float* scores, void* stream) {
  return run_estimate(kv, q, kmin, kmax, page_table, seq_lens, scores, true,
                      stream, "quest_estimate_heads");
}

QUEST_API quest_status quest_union_pages(const quest_paged_kv* kv,
                                         const int32_t* sel_heads,
                                         int32_t k_pages, int32_t* sel_union,
                                         void* stream) {
  const char* fn = "quest_union_pages";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(sel_heads, aligned4(sel_heads));
  REQUIRE_PTR(sel_union, aligned4(sel_union));
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  const int64_t G = kv->num_q_heads / kv->num_kv_heads;
  if (G * k_pages > (int64_t)1 << 30)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: G * k_pages too large", fn);
  if (kv->max_pages_per_seq > quest::kTopkMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq %d > %d", fn,
                kv->max_pages_per_seq, quest::kTopkMaxPages);
  return hip_status(quest::launch_union(*kv, sel_heads, k_pages, sel_union,
                                        static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_topk_pages_ex(const quest_paged_kv* kv,
                                           const float* scores,
                                           const int32_t* seq_lens,
                                           int32_t k_pages, int32_t n_sink,
                                           int32_t n_local, int32_t* sel_pages,
                                           void* stream) {
  const char* fn = "quest_topk_pages_ex";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(scores, aligned4(scores));
  REQUIRE_PTR(seq_lens, aligned4(seq_lens));
  REQUIRE_PTR(sel_pages, aligned4(sel_pages));
  if ((s = check_topk_counts(k_pages, n_sink, n_local, fn)) != QUEST_OK) return s;
  if (kv->max_pages_per_seq > quest::kTopkMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq %d > %d", fn,
                kv->max_pages_per_seq, quest::kTopkMaxPages);
  return hip_status(quest::launch_topk(*kv, scores, seq_lens, k_pages, n_sink,
                                       n_local, sel_pages,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_topk_pages(const quest_paged_kv* kv,
                                        const float* scores,
                                        const int32_t* seq_lens,
                                        int32_t k_pages, int32_t* sel_pages,
                                        void* stream) {
  const quest_status s =
      quest_topk_pages_ex(kv, scores, seq_lens, k_pages, 0, 0, sel_pages, stream);
  if (s != QUEST_OK) retag(g_last_error, "quest_topk_pages_ex", "quest_topk_pages");
  return s;
}

QUEST_API quest_status quest_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* sel_pages, int32_t k_pages, float sm_scale, float* out,
    void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "quest_sparse_decode_attn";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(sel_pages, aligned4(sel_pages));
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  return run_attention(kv, q, k_pool, v_pool, page_table, seq_lens, sel_pages,
                       k_pages, sm_scale, out, workspace, workspace_bytes,
                       stream, fn);
}

QUEST_API quest_status quest_union_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* sel_heads, int32_t k_pages, float sm_scale, int32_t* sel_union,
    float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "quest_union_sparse_decode_attn";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(sel_heads, aligned4(sel_heads));
  REQUIRE_PTR(sel_union, aligned4(sel_union));
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  const int64_t G = kv->num_q_heads / kv->num_kv_heads;
  if (G * k_pages > quest::kUnionListMax)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: G * k_pages = %lld > %d", fn,
                (long long)(G * k_pages), quest::kUnionListMax);
  if (kv->max_pages_per_seq > quest::kTopkMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq %d > %d", fn,
                kv->max_pages_per_seq, quest::kTopkMaxPages);
  s = check_attention_workspace(kv, (int)(G * k_pages), workspace, workspace_bytes, fn);
  if (s != QUEST_OK) return s;
  return hip_status(quest::launch_union_attention(*kv, q, k_pool, v_pool, page_table,
                                                  seq_lens, sel_heads, k_pages, sm_scale,
                                                  sel_union, out, workspace,
                                                  static_cast<hipStream_t>(stream)),
                    fn);
}

static quest_status run_topk_attention(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* workspace,
    size_t workspace_bytes, void* stream, bool merge, const char* fn) {
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(scores, aligned4(scores));
  REQUIRE_PTR(sel_pages, aligned4(sel_pages));
  if ((s = check_topk_counts(k_pages, n_sink, n_local, fn)) != QUEST_OK) return s;
  if (kv->max_pages_per_seq > quest::kTopkAttnMaxPages || k_pages > quest::kTopkAttnMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq and k_pages must be <= %d",
                fn, quest::kTopkAttnMaxPages);
  const size_t need = quest::attention_workspace_bytes(*kv, k_pages);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(QUEST_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu",
                  fn, need, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace))
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `workspace` is misaligned", fn);
  }
  return hip_status(quest::launch_topk_attention(
                        *kv, q, k_pool, v_pool, page_table, seq_lens, scores,
                        k_pages, n_sink, n_local, sm_scale, sel_pages, out,
                        workspace, static_cast<hipStream_t>(stream), merge),
                    fn);
}

QUEST_API quest_status quest_topk_sparse_decode_attn_ex(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  return run_topk_attention(kv, q, k_pool, v_pool, page_table, seq_lens, scores,
                            k_pages, n_sink, n_local, sm_scale, sel_pages, out,
                            workspace, workspace_bytes, stream, true,
                            "quest_topk_sparse_decode_attn_ex");
}

QUEST_API quest_status quest_topk_sparse_decode_attn_splits(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  return run_topk_attention(kv, q, k_pool, v_pool, page_table, seq_lens, scores,
                            k_pages, n_sink, n_local, sm_scale, sel_pages, out,
                            workspace, workspace_bytes, stream, false,
                            "quest_topk_sparse_decode_attn_splits");
}

QUEST_API quest_status quest_topk_sparse_decode_attn_noalloc(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* stream) {
  const char* fn = "quest_topk_sparse_decode_attn_noalloc";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(scores, aligned4(scores));
  REQUIRE_PTR(sel_pages, aligned4(sel_pages));
  if ((s = check_topk_counts(k_pages, n_sink, n_local, fn)) != QUEST_OK) return s;
  if (kv->max_pages_per_seq > quest::kTopkAttnMaxPages || k_pages > quest::kTopkAttnMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq and k_pages must be <= %d",
                fn, quest::kTopkAttnMaxPages);
  const size_t need = quest::attention_workspace_bytes(*kv, k_pages);
  if (need > quest::kNoAllocScratchBytes)
    return fail(QUEST_ERR_UNSUPPORTED,
                "%s: this geometry needs %zu bytes of split scratch; the "
                "allocation-free entry point holds %zu bytes per GPU (use "
                "quest_topk_sparse_decode_attn_ex with a workspace)",
                fn, need, quest::kNoAllocScratchBytes);
  return hip_status(quest::launch_topk_attention_noalloc(
                        *kv, q, k_pool, v_pool, page_table, seq_lens, scores,
                        k_pages, n_sink, n_local, sm_scale, sel_pages, out,
                        static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_merge_attn_splits(const quest_paged_kv* kv,
                                               int32_t k_pages,
                                               const void* workspace,
                                               size_t workspace_bytes,
                                               float* out, void* stream) {
  const char* fn = "quest_merge_attn_splits";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  REQUIRE_PTR(out, aligned4(out));
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  if (kv->max_pages_per_seq > quest::kTopkAttnMaxPages || k_pages > quest::kTopkAttnMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq and k_pages must be <= %d",
                fn, quest::kTopkAttnMaxPages);
  const size_t need = quest::attention_workspace_bytes(*kv, k_pages);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(QUEST_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu",
                  fn, need, workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned16(workspace))
      return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `workspace` is misaligned", fn);
  }
  return hip_status(quest::launch_topk_attention_merge(
                        *kv, k_pages, const_cast<void*>(workspace), out,
                        static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_topk_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, float sm_scale, int32_t* sel_pages,
    float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const quest_status s = quest_topk_sparse_decode_attn_ex(
      kv, q, k_pool, v_pool, page_table, seq_lens, scores, k_pages, 0, 0,
      sm_scale, sel_pages, out, workspace, workspace_bytes, stream);
  if (s != QUEST_OK)
    retag(g_last_error, "quest_topk_sparse_decode_attn_ex",
          "quest_topk_sparse_decode_attn");
  return s;
}

QUEST_API quest_status quest_decode_attn(const quest_paged_kv* kv,
                                         const void* q, const void* k_pool,
                                         const void* v_pool,
                                         const int32_t* page_table,
                                         const int32_t* seq_lens,
                                         float sm_scale, float* out,
                                         void* workspace,
                                         size_t workspace_bytes, void* stream) {
  const char* fn = "quest_decode_attn";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  return run_attention(kv, q, k_pool, v_pool, page_table, seq_lens, nullptr,
                       kv->max_pages_per_seq, sm_scale, out, workspace,
                       workspace_bytes, stream, fn);
}

QUEST_API quest_status quest_append_decode_attn(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin, void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, const void* k_new,
    const void* v_new, const void* q, float sm_scale, float* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* fn = "quest_append_decode_attn";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  REQUIRE_PTR(kmin, aligned16(kmin));
  REQUIRE_PTR(kmax, aligned16(kmax));
  REQUIRE_PTR(k_new, aligned16(k_new));
  REQUIRE_PTR(v_new, aligned16(v_new));
  const quest::AttnAppend ap{static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool),
                             static_cast<uint16_t*>(kmin), static_cast<uint16_t*>(kmax),
                             static_cast<const uint16_t*>(k_new),
                             static_cast<const uint16_t*>(v_new)};
  return run_attention(kv, q, k_pool, v_pool, page_table, seq_lens, nullptr,
                       kv->max_pages_per_seq, sm_scale, out, workspace,
                       workspace_bytes, stream, fn, &ap);
}

QUEST_API quest_status quest_sparse_decode_step(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const void* kmin, const void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, int32_t k_pages,
    float sm_scale, float* scores, int32_t* sel_pages, float* out,
    void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "quest_sparse_decode_step";
  quest_status s = check_attention_common(kv, q, k_pool, v_pool, page_table,
                                          seq_lens, sm_scale, out, fn);
  if (s != QUEST_OK) return s;
  if (!kFusedStepEnabled)
    return fail(QUEST_ERR_UNSUPPORTED,
                "%s: the one-launch step is switched off (its "
                "kernel did not complete on gfx950; cause not yet found) -- "
                "use quest_estimate + quest_topk_pages + "
                "quest_sparse_decode_attn", fn);
  REQUIRE_PTR(kmin, aligned16(kmin));
  REQUIRE_PTR(kmax, aligned16(kmax));
  REQUIRE_PTR(scores, aligned4(scores));
  REQUIRE_PTR(sel_pages, aligned4(sel_pages));
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  if (kv->max_pages_per_seq > quest::kStepMaxPages)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: max_pages_per_seq %d > %d", fn,
                kv->max_pages_per_seq, quest::kStepMaxPages);
  if (kv->page_size != quest::kTileRows)
    return fail(QUEST_ERR_UNSUPPORTED, "%s: 16-token pages only", fn);
  const size_t need = quest::step_workspace_bytes(*kv, k_pages);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(QUEST_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %zu bytes, got %zu",
                fn, need, workspace == nullptr ? (size_t)0 : workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `workspace` must be 256-byte aligned", fn);
  return hip_status(quest::launch_step(*kv, q, k_pool, v_pool, kmin, kmax,
                                       page_table, seq_lens, k_pages, sm_scale,
                                       scores, sel_pages, out, workspace,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

QUEST_API quest_status quest_step_workspace_size(const quest_paged_kv* kv,
                                                 int32_t k_pages, size_t* bytes) {
  const char* fn = "quest_step_workspace_size";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  if (bytes == nullptr)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `bytes` is NULL", fn);
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  *bytes = quest::step_workspace_bytes(*kv, k_pages);
  return ok();
}

QUEST_API quest_status quest_workspace_size(const quest_paged_kv* kv,
                                            int32_t k_pages, size_t* bytes) {
  const char* fn = "quest_workspace_size";
  quest_status s = check_kv(kv, fn);
  if (s != QUEST_OK) return s;
  if ((s = check_group(kv, fn)) != QUEST_OK) return s;
  if (bytes == nullptr)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: `bytes` is NULL", fn);
  if (k_pages < 1)
    return fail(QUEST_ERR_INVALID_ARGUMENT, "%s: k_pages must be >= 1", fn);
  *bytes = quest::attention_workspace_bytes(*kv, k_pages);
  return ok();
}

QUEST_API quest_status quest_host_device_pointer(const void* host_ptr,
                                                 void** device_ptr) {
  const char* fn = "quest_host_device_pointer";
  REQUIRE_PTR(host_ptr, true);
  REQUIRE_PTR(device_ptr, true);
  void* dev = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&dev, const_cast<void*>(host_ptr), 0);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear it: the caller's next HIP call must not see it
    return fail(QUEST_ERR_HIP, "%s: %s (is the buffer pinned host memory?)", fn,
                hipGetErrorString(e));
  }
  *device_ptr = dev;
  return ok();
}

QUEST_API quest_status quest_stream_read_probe(const void* buf, size_t bytes,
                                               uint32_t* sink, void* stream) {
  const char* fn = "quest_stream_read_probe";
  REQUIRE_PTR(buf, aligned16(buf));
  REQUIRE_PTR(sink, aligned4(sink));
  if (bytes == 0 || bytes % 16 != 0)
    return fail(QUEST_ERR_INVALID_ARGUMENT,
                "%s: bytes (%zu) must be a positive multiple of 16", fn, bytes);
  return hip_status(
      quest::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)),
      fn);
}

QUEST_API const char* quest_status_string(quest_status status) {
  // Callers across the C ABI may pass any int: read the argument's bytes as
  // an int rather than as the enum (a value outside the enumerators' range
  // is undefined behaviour for a C++ enum).
  int code = 0;
  static_assert(sizeof(code) == sizeof(status), "quest_status is int-sized");
  std::memcpy(&code, &status, sizeof(code));
  switch (code) {
    case QUEST_OK: return "ok";
    case QUEST_ERR_INVALID_ARGUMENT: return "invalid argument";
    case QUEST_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case QUEST_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QUEST_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

QUEST_API const char* quest_last_error(void) { return g_last_error; }

}  // extern "C"
