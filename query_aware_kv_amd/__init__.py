"""Quest decode-step hot path for AMD Instinct MI355X (gfx950).

The computation lives in libquest.so (hand-written HIP kernels behind a C
ABI, declared in include/quest.h).  This package is its Python binding:
every entry point under its C name, plus the step compositions on
preallocated buffers -- `SparseDecodeStep` (estimate -> Top-K -> sparse
attention, optionally appending the step's token first), `UnionDecodeStep`
(per-head Top-K and the group's union) and `DenseDecode`.  PyTorch only
provides device memory and the stream.
"""
from __future__ import annotations

import math

import torch

from ._abi import (  # noqa: F401
    LIB, LIB_PATH, HostPool, PagedKV, QuestError, QUEST_BF16, QUEST_F16, QUEST_OK,
    QUEST_ERR_HIP, QUEST_ERR_INVALID_ARGUMENT, QUEST_ERR_UNSUPPORTED,
    QUEST_ERR_WORKSPACE_TOO_SMALL, paged_kv, paged_kv_like,
    quest_decode_attn, quest_estimate, quest_sparse_decode_attn,
    quest_sparse_decode_step, quest_step_workspace_size,
    quest_append_estimate, quest_append_decode_attn, quest_estimate_heads,
    quest_union_pages, quest_union_sparse_decode_attn, UNION_LIST_MAX,
    quest_stream_read_probe, quest_topk_pages, quest_topk_pages_ex,
    quest_topk_sparse_decode_attn, quest_topk_sparse_decode_attn_ex,
    quest_topk_sparse_decode_attn_splits, quest_merge_attn_splits,
    quest_topk_sparse_decode_attn_noalloc,
    quest_update_page_meta,
    quest_workspace_size,
)

HEAD_DIM = 128
PAGE_SIZE = 16


def default_sm_scale(head_dim: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(head_dim)


def alloc_workspace(kv: PagedKV, k_pages: int, device="cuda") -> torch.Tensor:
    """Attention workspace: per-split partial results, whose contents on
    entry do not matter (allocated zeroed all the same)."""
    n = quest_workspace_size(kv, k_pages)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def host_pool_like(pool: torch.Tensor) -> HostPool:
    """A pinned host copy of a K or V pool, for the kernels to read in place
    (only the pages a call uses cross the host link)."""
    t = torch.empty(pool.shape, dtype=pool.dtype, pin_memory=True)
    t.copy_(pool)
    return HostPool(t)


def alloc_meta(kv: PagedKV, device="cuda"):
    shape = (kv.num_pool_pages, kv.num_kv_heads, kv.head_dim)
    return (torch.empty(shape, dtype=kv.torch_dtype, device=device),
            torch.empty(shape, dtype=kv.torch_dtype, device=device))


TOPK_ATTN_MAX_PAGES = 8192
SELECT_MODES = ("auto", "attention", "separate")
# With more (request, kv-head) rows than this, a separate Top-K launch (one
# selection per row) beats selecting in every attention workgroup (one per
# row and split): measured on the 32 x 32-head ragged batch (1024 rows).
AUTO_ATTENTION_MAX_ROWS = 256


class SparseDecodeStep:
    """Buffers and call sequence of one sparse decode step for a fixed
    geometry: quest_estimate, then the Top-K and the sparse attention.
    ``select`` says where the Top-K runs:

    - "attention": inside the attention launch
      (quest_topk_sparse_decode_attn_ex: every workgroup of a row selects
      the row's pages itself, so no selection crosses memory);
    - "separate": its own launch (quest_topk_pages_ex, one workgroup per
      row), then quest_sparse_decode_attn;
    - "auto" (default): "attention" for up to 256 (request, kv-head) rows,
      "separate" beyond.

    "attention" needs max_pages_per_seq <= 8192 and falls back to
    "separate" beyond it.  ``n_sink`` / ``n_local`` force the first / last
    pages of every row into the selection (0, 0: plain Top-K).
    """

    def __init__(self, kv: PagedKV, k_pages: int, sm_scale: float | None = None,
                 device="cuda", select: str = "auto", n_sink: int = 0,
                 n_local: int = 0):
        if select not in SELECT_MODES:
            raise ValueError(f"select must be one of {SELECT_MODES}, got {select!r}")
        self.kv = kv
        self.k_pages = int(k_pages)
        self.n_sink, self.n_local = int(n_sink), int(n_local)
        self.sm_scale = default_sm_scale(kv.head_dim) if sm_scale is None else sm_scale
        B, Hq, Hkv = kv.batch, kv.num_q_heads, kv.num_kv_heads
        self.scores = torch.empty(B, Hkv, kv.max_pages_per_seq,
                                  dtype=torch.float32, device=device)
        self.sel = torch.empty(B, Hkv, self.k_pages, dtype=torch.int32,
                               device=device)
        self.out = torch.empty(B, Hq, kv.head_dim, dtype=torch.float32,
                               device=device)
        self.workspace = alloc_workspace(kv, self.k_pages, device)
        if select == "auto":
            select = "attention" if B * Hkv <= AUTO_ATTENTION_MAX_ROWS else "separate"
        fits = kv.max_pages_per_seq <= TOPK_ATTN_MAX_PAGES and \
            self.k_pages <= TOPK_ATTN_MAX_PAGES
        self.select = select if fits else "separate"

    def _select_attend(self, q, k_pool, v_pool, page_table, seq_lens, stream):
        if self.select == "attention":
            quest_topk_sparse_decode_attn_ex(
                self.kv, q, k_pool, v_pool, page_table, seq_lens, self.scores,
                self.k_pages, self.n_sink, self.n_local, self.sm_scale,
                self.sel, self.out, self.workspace, stream)
            return self.out
        quest_topk_pages_ex(self.kv, self.scores, seq_lens, self.k_pages,
                            self.n_sink, self.n_local, self.sel, stream)
        quest_sparse_decode_attn(self.kv, q, k_pool, v_pool, page_table,
                                 seq_lens, self.sel, self.k_pages,
                                 self.sm_scale, self.out, self.workspace,
                                 stream)
        return self.out

    def __call__(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                 stream=None) -> torch.Tensor:
        quest_estimate(self.kv, q, kmin, kmax, page_table, seq_lens,
                       self.scores, stream)
        return self._select_attend(q, k_pool, v_pool, page_table, seq_lens, stream)

    def append_step(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                    k_new, v_new, stream=None) -> torch.Tensor:
        """One generated token per request: append k_new / v_new at position
        seq_lens - 1 (which already counts it) together with the estimate
        (quest_append_estimate), then select and attend."""
        quest_append_estimate(self.kv, k_pool, v_pool, kmin, kmax, page_table,
                              seq_lens, k_new, v_new, q, self.scores, stream)
        return self._select_attend(q, k_pool, v_pool, page_table, seq_lens, stream)


class UnionDecodeStep:
    """The GQA group rule of per-head selection + union ("Guide to Quest",
    Best Practices 2): quest_estimate_heads, quest_topk_pages_ex per query
    head, then attention over the union of a group's lists (up to
    G * k_pages pages per kv-head, shared by the group's heads).  The union
    is built inside the attention launch (quest_union_sparse_decode_attn)
    when G * k_pages <= UNION_LIST_MAX, else by quest_union_pages before
    quest_sparse_decode_attn; `fused=False` takes the second path always.
    Both give the same bits."""

    def __init__(self, kv: PagedKV, k_pages: int, sm_scale: float | None = None,
                 device="cuda", n_sink: int = 0, n_local: int = 0,
                 fused: bool | None = None):
        self.kv = kv
        self.k_pages = int(k_pages)
        self.n_sink, self.n_local = int(n_sink), int(n_local)
        self.sm_scale = default_sm_scale(kv.head_dim) if sm_scale is None else sm_scale
        B, Hq, Hkv = kv.batch, kv.num_q_heads, kv.num_kv_heads
        self.group = Hq // Hkv
        # per-head rows: the same geometry seen with one row per query head
        self.kv_heads = paged_kv(B, Hq, Hq, kv.num_pool_pages,
                                 kv.max_pages_per_seq, kv.torch_dtype,
                                 kv.head_dim, kv.page_size)
        self.scores = torch.empty(B, Hq, kv.max_pages_per_seq,
                                  dtype=torch.float32, device=device)
        self.sel_heads = torch.empty(B, Hq, self.k_pages, dtype=torch.int32,
                                     device=device)
        self.sel = torch.empty(B, Hkv, self.group * self.k_pages,
                               dtype=torch.int32, device=device)
        self.out = torch.empty(B, Hq, kv.head_dim, dtype=torch.float32,
                               device=device)
        self.workspace = alloc_workspace(kv, self.group * self.k_pages, device)
        fits = self.group * self.k_pages <= UNION_LIST_MAX
        self.fused = fits if fused is None else bool(fused) and fits

    def __call__(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                 stream=None) -> torch.Tensor:
        quest_estimate_heads(self.kv, q, kmin, kmax, page_table, seq_lens,
                             self.scores, stream)
        quest_topk_pages_ex(self.kv_heads, self.scores, seq_lens, self.k_pages,
                            self.n_sink, self.n_local, self.sel_heads, stream)
        if self.fused:
            quest_union_sparse_decode_attn(self.kv, q, k_pool, v_pool, page_table,
                                           seq_lens, self.sel_heads, self.k_pages,
                                           self.sm_scale, self.sel, self.out,
                                           self.workspace, stream)
            return self.out
        quest_union_pages(self.kv, self.sel_heads, self.k_pages, self.sel,
                          stream)
        quest_sparse_decode_attn(self.kv, q, k_pool, v_pool, page_table,
                                 seq_lens, self.sel, self.group * self.k_pages,
                                 self.sm_scale, self.out, self.workspace,
                                 stream)
        return self.out


class FusedDecodeStep(SparseDecodeStep):
    """The same step as `SparseDecodeStep` in one launch
    (quest_sparse_decode_step).  Owns a zero-initialised workspace, which
    every call leaves zeroed again; use one instance per stream."""

    def __init__(self, kv: PagedKV, k_pages: int, sm_scale: float | None = None,
                 device="cuda"):
        super().__init__(kv, k_pages, sm_scale, device)
        n = quest_step_workspace_size(kv, self.k_pages)
        self.workspace = torch.zeros(max(n, 256), dtype=torch.uint8, device=device)

    def __call__(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                 stream=None) -> torch.Tensor:
        quest_sparse_decode_step(self.kv, q, k_pool, v_pool, kmin, kmax,
                                 page_table, seq_lens, self.k_pages,
                                 self.sm_scale, self.scores, self.sel,
                                 self.out, self.workspace, stream)
        return self.out

    def control_words(self) -> torch.Tensor:
        """The work-queue counters (ticket, exited, stalls): zero between
        calls, stalls zero always."""
        return self.workspace[:12].view(torch.int32)


class DenseDecode:
    """Buffers of the dense baseline (quest_decode_attn) for a geometry."""

    def __init__(self, kv: PagedKV, sm_scale: float | None = None,
                 device="cuda"):
        self.kv = kv
        self.sm_scale = default_sm_scale(kv.head_dim) if sm_scale is None else sm_scale
        self.out = torch.empty(kv.batch, kv.num_q_heads, kv.head_dim,
                               dtype=torch.float32, device=device)
        self.workspace = alloc_workspace(kv, kv.max_pages_per_seq, device)

    def __call__(self, q, k_pool, v_pool, page_table, seq_lens,
                 stream=None) -> torch.Tensor:
        quest_decode_attn(self.kv, q, k_pool, v_pool, page_table, seq_lens,
                          self.sm_scale, self.out, self.workspace, stream)
        return self.out

    def append_step(self, q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                    k_new, v_new, stream=None) -> torch.Tensor:
        """Append the step's token (seq_lens already count it) and attend
        over every token, in one launch (quest_append_decode_attn)."""
        quest_append_decode_attn(self.kv, k_pool, v_pool, kmin, kmax, page_table,
                                 seq_lens, k_new, v_new, q, self.sm_scale, self.out,
                                 self.workspace, stream)
        return self.out
