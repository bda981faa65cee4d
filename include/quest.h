/*
 * quest.h -- C ABI of libquest.so: the decode-step hot path of Quest
 * (query-aware KV-cache page sparsity) for AMD Instinct MI355X (gfx950).
 *
 * Sources (page title, section / equation):
 *   [G] "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs":
 *       §1 Offline Min-Max Key Vector Bounding Boxes (the min/max equation),
 *       §2 Fast Query-Aware Logit Upper-Bound Estimation (the bound),
 *       §3 Top-K Page Selection and Sparse FlashAttention Dispatch,
 *       "The Memory Bandwidth Bottleneck of Long-Context Decoding"
 *       (the attention equation), Implementation Steps 1-3 (the interface:
 *       page append, bound estimation, page selection, sparse forward).
 *   [Q] "Quest: Query-Aware Sparsity for Efficient Long-Context LLM
 *       Inference" (paper summary): Summary, Key points.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array arguments are DEVICE pointers to row-major, contiguous memory,
 *   16-byte aligned (the kernels read and write 16 bytes per lane).  The K/V
 *   pools may instead be pinned host memory seen through its device address
 *   (quest_host_device_pointer).  The
 *   caller allocates and owns every buffer; the library allocates nothing,
 *   keeps no state between calls, and may be called from several host
 *   threads on different streams.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call only enqueues work on it and returns; the status reports the
 *   host-side checks and the launch, never the kernels' completion.
 * - Device-side VALUES are not validated, but they cannot cause an
 *   out-of-bounds read: a page id outside [0, num_pool_pages) is treated as
 *   an absent page (never read; its score is -inf), and a length above
 *   max_pages_per_seq * page_size is clamped to it.
 * - Slots of a page past the sequence's last token, and pool pages no
 *   request owns, may hold any bits (NaN included): they are never used as
 *   values.
 * - Shapes (d = head_dim = 128, S = page_size = 16 or 32, G = Hq / Hkv):
 *     k_pool, v_pool  [num_pool_pages][Hkv][S][d]   (dtype)
 *     kmin, kmax      [num_pool_pages][Hkv][d]      (dtype)
 *     page_table      int32 [batch][max_pages_per_seq]; logical page j of
 *                     request b lives in pool page page_table[b][j]
 *     seq_lens        int32 [batch]; L_b tokens, n_b = ceil(L_b / S) pages;
 *                     L_b = 0 is allowed (an empty request)
 *     q               [batch][Hq][d]                (dtype)
 *     scores          float32 [batch][Hkv][max_pages_per_seq]
 *     sel_pages       int32 [batch][Hkv][k_pages]
 *     out             float32 [batch][Hq][d]
 *   Query head h reads kv-head h / G.
 * - Errors: a non-OK status means nothing was enqueued (except
 *   QUEST_ERR_HIP, which reports a failed launch); quest_last_error() then
 *   returns a thread-local message naming the argument or the HIP error.
 */
#ifndef QUEST_H_
#define QUEST_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QUEST_API __attribute__((visibility("default")))

typedef enum quest_status {
  QUEST_OK = 0,
  QUEST_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, bad count */
  QUEST_ERR_UNSUPPORTED = 2,      /* shape or dtype the library has no kernel for */
  QUEST_ERR_WORKSPACE_TOO_SMALL = 3,
  QUEST_ERR_HIP = 4               /* the HIP runtime reported an error */
} quest_status;

typedef enum quest_dtype {
  QUEST_F16 = 0, /* IEEE binary16 */
  QUEST_BF16 = 1 /* bfloat16 */
} quest_dtype;

/* Geometry of one paged KV cache (one layer).  Host memory. */
typedef struct quest_paged_kv {
  int32_t batch;             /* requests, >= 1 */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv, >= 1 */
  int32_t head_dim;          /* d: must be 128 */
  int32_t page_size;         /* S: 16 or 32 ("Guide to Quest", Best Practices 1) */
  int32_t num_pool_pages;    /* pages in k_pool / v_pool / kmin / kmax */
  int32_t max_pages_per_seq; /* columns of page_table and scores */
  int32_t dtype;             /* quest_dtype of q, K, V, kmin, kmax */
} quest_paged_kv;

/*
 * Page metadata: per-page, per-channel min and max of the keys.
 * [G] §1 (min/max equation): Kmin[p] = min_t K[p,t], Kmax[p] = max_t K[p,t]
 * over the page's valid tokens, stored in K's dtype.  Min/max only select
 * an input, so the result is exact; signed zeros order as -0 < +0.
 *
 * Two modes:
 *  - Rebuild (k_new == NULL, v_new == NULL): for each request b fold the
 *    tokens [f_b, L_b) already in k_pool into their pages' boxes, where
 *    f_b = first_token[b] (first_token == NULL means f_b = 0 for all b).
 *    A page whose slot 0 lies in [f_b, L_b) is rebuilt from its valid
 *    tokens; a page entered in mid-page is widened.  first_token all zero
 *    is a full rebuild.  k_pool and v_pool are not written.
 *  - Append (k_new, v_new non-NULL, first_token must be NULL): each request
 *    appends one token at position L_b - 1 (seq_lens already count it):
 *    k_new/v_new [batch][Hkv][d] are written into slot (L_b-1) % S of
 *    logical page (L_b-1) / S, then folded into that page's box ([G] §1:
 *    the box forms as its page forms, here one generated token at a time; a
 *    token in slot 0 starts a new box).  Requests with L_b = 0 are skipped.
 * kmin/kmax of pages outside the folded range are left untouched.
 */
QUEST_API quest_status quest_update_page_meta(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin,
    void* kmax, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* first_token, const void* k_new, const void* v_new,
    void* stream);

/*
 * Query-aware page estimate.  [G] §2 (upper-bound inequality):
 *   scores[b][g][j] = sum_{h in group g} sum_i max(q[b][h][i] * kmin[p][g][i],
 *                                                 q[b][h][i] * kmax[p][g][i]),
 *   p = page_table[b][j], for j < n_b; scores[b][g][j] = -inf for
 *   n_b <= j < max_pages_per_seq.
 * Unscaled (no 1/sqrt(d)); a GQA group's score is the sum of its G query
 * heads' bounds.  The boxes must satisfy kmin <= kmax in every channel, as
 * quest_update_page_meta writes them: each term is then evaluated as
 * q_i * kmax_i for q_i >= 0 and q_i * kmin_i otherwise, which is the max.
 * Products are exact in float32 for fp16/bf16 inputs whenever the product
 * is a normal float32 number (16-bit subnormal inputs are not flushed);
 * the sum rounds in float32.
 */
QUEST_API quest_status quest_estimate(
    const quest_paged_kv* kv, const void* q, const void* kmin,
    const void* kmax, const int32_t* page_table, const int32_t* seq_lens,
    float* scores, void* stream);

/*
 * quest_update_page_meta in append mode followed by quest_estimate, in one
 * launch, with the same results bit for bit: each request appends token
 * L_b - 1 (k_new / v_new [batch][Hkv][d], written into k_pool / v_pool at
 * slot (L_b - 1) % S of logical page (L_b - 1) / S, folded into that page's
 * box in kmin / kmax -- [G] §1, the box forms as its page forms), and the
 * scores are those of the updated boxes.  Requests with L_b = 0 append
 * nothing.  The decode step of one layer becomes this call plus
 * quest_topk_sparse_decode_attn.  The page a request appends into must be
 * its own: no other request's row may list it (its box and slot are
 * written while the other rows are read).
 */
QUEST_API quest_status quest_append_estimate(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin, void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, const void* k_new,
    const void* v_new, const void* q, float* scores, void* stream);

/*
 * Per-query-head estimate.  [G] §2 upper-bound inequality for each query
 * head h against the boxes of its kv-head g = h / G, as [G] Best Practices 2
 * asks for before the union of the heads' selections:
 *   scores[b][h][j] = sum_i max(q[b][h][i] * kmin[p][g][i],
 *                               q[b][h][i] * kmax[p][g][i]),
 * p = page_table[b][j], j < n_b; -inf for n_b <= j < max_pages_per_seq.
 * `scores` is float32 [batch][Hq][max_pages_per_seq]; each box is read once
 * for the G heads.  Arithmetic as quest_estimate (whose group sum these
 * rows add up to, up to float32 rounding).
 */
QUEST_API quest_status quest_estimate_heads(
    const quest_paged_kv* kv, const void* q, const void* kmin,
    const void* kmax, const int32_t* page_table, const int32_t* seq_lens,
    float* scores, void* stream);

/*
 * Union of a GQA group's per-head selections.  [G] Best Practices 2: the
 * kv-head loads the union of its query heads' Top-K pages once and every
 * head of the group attends all of them.  sel_heads is int32
 * [batch][Hq][k_pages] (each query head's list, as written by
 * quest_topk_pages(_ex) run on quest_estimate_heads' scores with a
 * descriptor whose num_kv_heads = num_q_heads); sel_union is int32
 * [batch][Hkv][G * k_pages]: for each (b, g) the distinct pages listed by
 * heads g*G .. g*G+G-1, ascending, then -1.  Entries outside
 * [0, max_pages_per_seq) are ignored.  Pass sel_union to
 * quest_sparse_decode_attn with k_pages' = G * k_pages.  Requires
 * max_pages_per_seq <= 32768.
 */
QUEST_API quest_status quest_union_pages(
    const quest_paged_kv* kv, const int32_t* sel_heads, int32_t k_pages,
    int32_t* sel_union, void* stream);

/*
 * Top-K page selection.  [G] §3: keep the k_pages pages with the highest
 * scores; Implementation Step 2: a request with n_b <= k_pages keeps all of
 * its pages.  For each (b, g) row the kept set is the first min(k_pages, n_b)
 * logical pages in the order (score descending, page index ascending), with
 * -0 == +0; sel_pages[b][g] lists it in ASCENDING page order, then -1 up to
 * k_pages.  Scores must not be NaN.  1 <= k_pages; max_pages_per_seq <=
 * 32768.
 */
QUEST_API quest_status quest_topk_pages(
    const quest_paged_kv* kv, const float* scores, const int32_t* seq_lens,
    int32_t k_pages, int32_t* sel_pages, void* stream);

/*
 * Top-K with forced pages.  [G] §3 and Implementation Step 2: the first
 * pages (attention sinks) and the most recent pages (the local window) are
 * kept unconditionally and the rest of the budget goes to the highest
 * bounds among the other pages.  For a row with n_b > k_pages the kept set
 * is pages j < n_sink, pages j >= n_b - n_local, and the first
 * k_pages - n_sink - n_local of the remaining pages in the order (score
 * descending, page index ascending); a row with n_b <= k_pages keeps all of
 * its pages.  Output as for quest_topk_pages (ascending, -1 padded).
 * Requires 0 <= n_sink, 0 <= n_local and n_sink + n_local <= k_pages
 * (QUEST_ERR_INVALID_ARGUMENT otherwise), so every row keeps exactly
 * min(k_pages, n_b) pages; n_local = 0 means no window.  n_sink = n_local =
 * 0 is quest_topk_pages.  Scores of forced pages are not read as values.
 */
QUEST_API quest_status quest_topk_pages_ex(
    const quest_paged_kv* kv, const float* scores, const int32_t* seq_lens,
    int32_t k_pages, int32_t n_sink, int32_t n_local, int32_t* sel_pages,
    void* stream);

/*
 * Sparse exact decode attention over the selected pages.  [Q] Summary and
 * [G] §3: attention runs only over the kept pages' tokens.  For query head
 * h (kv-head g = h / G) of request b, over the tokens t < v_j of every page
 * j >= 0 listed in sel_pages[b][g] (v_j = min(S, L_b - j*S)):
 *   out[b][h] = sum_t softmax(sm_scale * q[b][h].K_t)_t * V_t     (float32)
 * Entries equal to -1 are skipped; a row with no page yields zeros.  The
 * listed pages must be distinct and < n_b.  Accumulation is float32
 * (online softmax, split over pages, merged in float32).
 * `workspace` (device, >= quest_workspace_size(kv, k_pages) bytes) holds
 * per-split partial results; its contents on entry do not matter.  A
 * workspace serves one stream at a time.
 */
QUEST_API quest_status quest_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* sel_pages, int32_t k_pages, float sm_scale, float* out,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * quest_topk_pages followed by quest_sparse_decode_attn, in one launch (plus
 * the split merge): the same sel_pages bit for bit, and the same out up to
 * the float32 rounding of a different split and merge order (workgroups of
 * 8 waves here, 4 in quest_sparse_decode_attn).  Every
 * attention workgroup of a (request, kv-head) row recomputes the row's exact
 * Top-K from `scores` (float32 [batch][Hkv][max_pages_per_seq], e.g. from
 * quest_estimate) and keeps it in LDS, so no workgroup waits for another and
 * the selection makes no round trip through memory.  Requires
 * max_pages_per_seq <= 8192 and k_pages <= 8192.  Workspace as for
 * quest_sparse_decode_attn with the same k_pages.
 */
QUEST_API quest_status quest_topk_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, float sm_scale, int32_t* sel_pages,
    float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * quest_topk_pages_ex followed by quest_sparse_decode_attn in one launch
 * (plus the split merge); otherwise as quest_topk_sparse_decode_attn, whose
 * n_sink = n_local = 0 case it is.
 */
QUEST_API quest_status quest_topk_sparse_decode_attn_ex(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * quest_topk_sparse_decode_attn_ex in its two launches, for callers that
 * time them apart or put other work between them.  This call is the first:
 * the same Top-K and attention (sel_pages bit for bit as _ex), stopping
 * before the split merge -- each workgroup's partial result (running max,
 * softmax denominator, unnormalised output) stays in `workspace`, except
 * when the plan has a single split per row, in which case `out` is written
 * here directly.  quest_merge_attn_splits with the same kv, k_pages and
 * workspace then completes `out` ([Q] Summary, exact attention: the online
 * softmax merge is the last step of the same sum).  Arguments, limits and
 * errors as quest_topk_sparse_decode_attn_ex; the workspace must not be
 * reused between the two calls.
 */
QUEST_API quest_status quest_topk_sparse_decode_attn_splits(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * The second launch of quest_topk_sparse_decode_attn_ex: merges the split
 * partials that quest_topk_sparse_decode_attn_splits left in `workspace`
 * (same kv and k_pages) into out [batch][Hq][128] (float32); does nothing
 * when that plan has a single split (out is already written).  Same
 * workspace size rule; k_pages and max_pages_per_seq <= 8192.
 */
QUEST_API quest_status quest_merge_attn_splits(const quest_paged_kv* kv,
                                               int32_t k_pages,
                                               const void* workspace,
                                               size_t workspace_bytes,
                                               float* out, void* stream);

/*
 * quest_topk_sparse_decode_attn_ex without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The split partials
 * go to a scratch array inside the library, 8 MiB (8388608 bytes) per GPU,
 * held from the library's load until the process ends; the entry point
 * itself calls no hipMalloc, hipFree or other allocating routine.  Outputs
 * (sel_pages, out) are bit-identical to quest_topk_sparse_decode_attn_ex.
 * Geometries whose partials exceed the scratch (quest_workspace_size(kv,
 * k_pages) > 8 MiB) are refused with QUEST_ERR_UNSUPPORTED before any
 * launch.  Every call on one GPU shares that GPU's scratch and leaves its
 * partials there: calls that may overlap on one GPU (other streams, other
 * host threads) race and must not be issued.  Other arguments, limits and
 * errors as quest_topk_sparse_decode_attn_ex.
 */
QUEST_API quest_status quest_topk_sparse_decode_attn_noalloc(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const float* scores, int32_t k_pages, int32_t n_sink, int32_t n_local,
    float sm_scale, int32_t* sel_pages, float* out, void* stream);

/*
 * Dense decode attention over all L_b tokens (the in-library baseline).
 * "The Memory Bandwidth Bottleneck of Long-Context Decoding" in [G]:
 *   out[b][h] = softmax(sm_scale * q K^T) V over every token of request b.
 * Same kernels, arithmetic and workspace rules as the sparse call; the
 * workspace must hold quest_workspace_size(kv, max_pages_per_seq) bytes.
 */
QUEST_API quest_status quest_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    float sm_scale, float* out, void* workspace, size_t workspace_bytes,
    void* stream);

/*
 * quest_union_pages followed by quest_sparse_decode_attn over its output, in
 * one launch (+ the split merge), with the same results bit for bit ([G]
 * Best Practices 2: every query head of a group attends the union of the
 * group's per-head Top-K pages; [G] attention equation over their valid
 * tokens).  sel_heads is int32 [batch][Hq][k_pages] as for
 * quest_union_pages; sel_union, int32 [batch][Hkv][G * k_pages], receives
 * the union lists (ascending, then -1); out and the workspace
 * (quest_workspace_size(kv, G * k_pages) bytes) are those of
 * quest_sparse_decode_attn with k_pages' = G * k_pages.  Every workgroup of
 * a (request, kv-head) row builds the row's union in LDS, so the separate
 * union launch and its round trip go away.  Requires G * k_pages <= 4096
 * and max_pages_per_seq <= 32768 (QUEST_ERR_UNSUPPORTED otherwise).
 */
QUEST_API quest_status quest_union_sparse_decode_attn(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
    const int32_t* sel_heads, int32_t k_pages, float sm_scale, int32_t* sel_union,
    float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * quest_update_page_meta in append mode followed by quest_decode_attn, in
 * one launch (+ the split merge), with the same results bit for bit: each
 * request appends token L_b - 1 (k_new / v_new [batch][Hkv][d], written
 * into k_pool / v_pool at slot (L_b - 1) % S of logical page (L_b - 1) / S
 * and folded into that page's box in kmin / kmax -- [G] §1, the box forms
 * as its page forms), and the attention runs over all L_b tokens, the new
 * one included ([G] attention equation).  Requests with L_b = 0 append
 * nothing.  The decode step of a dense layer becomes this one call.  The
 * workspace must hold quest_workspace_size(kv, max_pages_per_seq) bytes.
 * As in quest_append_estimate, the page a request appends into must be its
 * own: no other request's row may list it.
 */
QUEST_API quest_status quest_append_decode_attn(
    const quest_paged_kv* kv, void* k_pool, void* v_pool, void* kmin, void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, const void* k_new,
    const void* v_new, const void* q, float sm_scale, float* out, void* workspace,
    size_t workspace_bytes, void* stream);

/*
 * One whole sparse decode step -- quest_estimate, quest_topk_pages and
 * quest_sparse_decode_attn -- in a single persistent launch, with the same
 * three outputs (scores, sel_pages, out) and the same arithmetic and tie
 * rules.  Each (request, kv-head) row's Top-K runs as soon as that row's
 * estimate is complete, overlapping the estimate and attention of other rows.
 * Requires max_pages_per_seq <= 8192 (QUEST_ERR_UNSUPPORTED otherwise).
 *
 * STATUS: switched off -- every call returns
 * QUEST_ERR_UNSUPPORTED before launching anything (its kernel did not
 * complete on gfx950 and the cause is not yet found).  Use the three
 * separate calls.
 *
 * `workspace` (device, >= quest_step_workspace_size(kv, k_pages) bytes) holds
 * work-queue counters, per-row flags and split partials.  Its bytes must be
 * ZERO before its first use (e.g. allocated zeroed); every call leaves the
 * counters at zero again.  A workspace serves one stream at a time: calls
 * that may overlap need their own workspaces.
 */
QUEST_API quest_status quest_sparse_decode_step(
    const quest_paged_kv* kv, const void* q, const void* k_pool,
    const void* v_pool, const void* kmin, const void* kmax,
    const int32_t* page_table, const int32_t* seq_lens, int32_t k_pages,
    float sm_scale, float* scores, int32_t* sel_pages, float* out,
    void* workspace, size_t workspace_bytes, void* stream);

/* Host only: workspace bytes quest_sparse_decode_step needs. */
QUEST_API quest_status quest_step_workspace_size(const quest_paged_kv* kv,
                                                 int32_t k_pages, size_t* bytes);

/* Host only: workspace bytes the attention calls need for k_pages selected
 * pages per row (pass max_pages_per_seq for quest_decode_attn). */
QUEST_API quest_status quest_workspace_size(const quest_paged_kv* kv,
                                            int32_t k_pages, size_t* bytes);

/*
 * Host-resident KV pools.  [G] (the introduction) keeps the full KV cache in
 * host or device memory and loads only the critical pages for the current
 * query.  k_pool and v_pool of quest_update_page_meta,
 * quest_sparse_decode_attn(_ex), quest_topk_sparse_decode_attn(_ex) and
 * quest_decode_attn may point to pinned host memory (allocated pinned, e.g.
 * with hipHostMalloc) through the device address this call returns: the
 * kernels then read, over the host link, only the 16-token tiles of the
 * pages they use, while kmin/kmax, scores and everything else stay in HBM.
 * Results are bit-identical to device-resident pools.  Host only; returns
 * QUEST_ERR_HIP if `host_ptr` is not pinned host memory.
 */
QUEST_API quest_status quest_host_device_pointer(const void* host_ptr,
                                                 void** device_ptr);

/*
 * Diagnostic, not part of the method: reads `bytes` (a positive multiple of
 * 16) of device memory at `buf` (16-byte aligned) once, as a plain streaming
 * read with 16-byte loads over the whole GPU.  Its time gives the HBM read
 * ceiling that the read-bound calls above are compared against.  `sink`
 * (device, 4-byte aligned, one uint32) is written only if the xor of all
 * loaded words equals 0x9e3779b9; its value means nothing.
 */
QUEST_API quest_status quest_stream_read_probe(const void* buf, size_t bytes,
                                               uint32_t* sink, void* stream);

/* Host only: static description of a status code. */
QUEST_API const char* quest_status_string(quest_status status);

/* Host only: detail of the last non-OK status on this thread ("" if none). */
QUEST_API const char* quest_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QUEST_H_ */
