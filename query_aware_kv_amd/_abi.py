"""ctypes binding of libquest.so: argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks their
dtype, device, shape and contiguity, and passes raw device pointers plus the
current HIP stream to the C entry point of the same name.  Every step of the
computation runs in the library's HIP kernels; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QUEST_LIB names another build of the same library (the host-sanitized one
# the ABI tests run against); by default the in-tree build.
LIB_PATH = os.environ.get("QUEST_LIB") or os.path.join(_HERE, "libquest.so")

QUEST_OK = 0
QUEST_ERR_INVALID_ARGUMENT = 1
QUEST_ERR_UNSUPPORTED = 2
QUEST_ERR_WORKSPACE_TOO_SMALL = 3
QUEST_ERR_HIP = 4

QUEST_F16 = 0
QUEST_BF16 = 1

_TORCH_DTYPE = {QUEST_F16: torch.float16, QUEST_BF16: torch.bfloat16}
_QUEST_DTYPE = {torch.float16: QUEST_F16, torch.bfloat16: QUEST_BF16}


class PagedKV(ctypes.Structure):
    """Mirror of ``quest_paged_kv`` (include/quest.h)."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


class QuestError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python query_aware_kv_amd/build.py` "
            "(or __graft_entry__.build()) first; there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int32
    KV = ctypes.POINTER(PagedKV)
    sig = {
        "quest_update_page_meta": [KV, P, P, P, P, P, P, P, P, P, P],
        "quest_estimate": [KV, P, P, P, P, P, P, P],
        "quest_topk_pages": [KV, P, P, I, P, P],
        "quest_sparse_decode_attn": [KV, P, P, P, P, P, P, I, ctypes.c_float,
                                     P, P, ctypes.c_size_t, P],
        "quest_decode_attn": [KV, P, P, P, P, P, ctypes.c_float, P, P,
                              ctypes.c_size_t, P],
        "quest_workspace_size": [KV, I, ctypes.POINTER(ctypes.c_size_t)],
        "quest_sparse_decode_step": [KV, P, P, P, P, P, P, P, I, ctypes.c_float,
                                     P, P, P, P, ctypes.c_size_t, P],
        "quest_step_workspace_size": [KV, I, ctypes.POINTER(ctypes.c_size_t)],
        "quest_topk_sparse_decode_attn": [KV, P, P, P, P, P, P, I, ctypes.c_float,
                                          P, P, P, ctypes.c_size_t, P],
        "quest_stream_read_probe": [P, ctypes.c_size_t, P, P],
        "quest_host_device_pointer": [P, ctypes.POINTER(ctypes.c_void_p)],
        "quest_topk_pages_ex": [KV, P, P, I, I, I, P, P],
        "quest_estimate_heads": [KV, P, P, P, P, P, P, P],
        "quest_append_estimate": [KV, P, P, P, P, P, P, P, P, P, P, P],
        "quest_append_decode_attn": [KV, P, P, P, P, P, P, P, P, P, ctypes.c_float,
                                     P, P, ctypes.c_size_t, P],
        "quest_union_pages": [KV, P, I, P, P],
        "quest_union_sparse_decode_attn": [KV, P, P, P, P, P, P, I, ctypes.c_float,
                                           P, P, P, ctypes.c_size_t, P],
        "quest_topk_sparse_decode_attn_ex": [KV, P, P, P, P, P, P, I, I, I,
                                             ctypes.c_float, P, P, P,
                                             ctypes.c_size_t, P],
        "quest_topk_sparse_decode_attn_splits": [KV, P, P, P, P, P, P, I, I, I,
                                                 ctypes.c_float, P, P, P,
                                                 ctypes.c_size_t, P],
        "quest_merge_attn_splits": [KV, I, P, ctypes.c_size_t, P, P],
        "quest_topk_sparse_decode_attn_noalloc": [KV, P, P, P, P, P, P, I, I, I,
                                                  ctypes.c_float, P, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.quest_status_string.argtypes = [ctypes.c_int]
    lib.quest_status_string.restype = ctypes.c_char_p
    lib.quest_last_error.argtypes = []
    lib.quest_last_error.restype = ctypes.c_char_p
    return lib


LIB = _load()


def _check(status: int) -> None:
    if status != QUEST_OK:
        raise QuestError(status, LIB.quest_last_error().decode())


class HostPool:
    """A K or V pool in pinned host memory, read by the kernels in place
    through its device address (only the pages a call uses cross the host
    link).  `tensor` must be a pinned CPU tensor, e.g. allocated with
    ``torch.empty(..., pin_memory=True)``."""

    def __init__(self, tensor: torch.Tensor):
        if tensor.device.type != "cpu" or not tensor.is_pinned():
            raise ValueError("HostPool needs a pinned CPU tensor")
        if not tensor.is_contiguous():
            raise ValueError("HostPool tensor must be contiguous")
        self.tensor = tensor
        dev = ctypes.c_void_p()
        _check(LIB.quest_host_device_pointer(ctypes.c_void_p(tensor.data_ptr()),
                                             ctypes.byref(dev)))
        self.device_ptr = int(dev.value)
        self.dtype, self.shape = tensor.dtype, tuple(tensor.shape)


def _ptr(t, name: str, dtype=None, shape=None, host_ok: bool = False):
    if t is None:
        return None
    if host_ok and isinstance(t, HostPool):
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        if shape is not None and t.shape != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got {t.shape}")
        return ctypes.c_void_p(t.device_ptr)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def paged_kv(batch: int, num_q_heads: int, num_kv_heads: int,
             num_pool_pages: int, max_pages_per_seq: int,
             dtype: torch.dtype, head_dim: int = 128,
             page_size: int = 16) -> PagedKV:
    if dtype not in _QUEST_DTYPE:
        raise ValueError(f"unsupported dtype {dtype}")
    return PagedKV(batch, num_q_heads, num_kv_heads, head_dim, page_size,
                   num_pool_pages, max_pages_per_seq, _QUEST_DTYPE[dtype])


def paged_kv_like(q: torch.Tensor, k_pool: torch.Tensor,
                  page_table: torch.Tensor) -> PagedKV:
    """Descriptor read off the tensors' shapes: q [B, Hq, d],
    k_pool [P, Hkv, S, d], page_table [B, max_pages]."""
    B, Hq, d = q.shape
    P, Hkv, S, d2 = k_pool.shape
    if d2 != d or page_table.shape[0] != B:
        raise ValueError("q, k_pool and page_table shapes disagree")
    return paged_kv(B, Hq, Hkv, P, page_table.shape[1], k_pool.dtype, d, S)


# --------------------------------------------------------------- entry points

def _pool_shape(kv):
    return (kv.num_pool_pages, kv.num_kv_heads, kv.page_size, kv.head_dim)


def _meta_shape(kv):
    return (kv.num_pool_pages, kv.num_kv_heads, kv.head_dim)


def quest_update_page_meta(kv: PagedKV, k_pool, v_pool, kmin, kmax,
                           page_table, seq_lens, first_token=None, k_new=None,
                           v_new=None, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    _check(LIB.quest_update_page_meta(
        ctypes.byref(kv),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(first_token, "first_token", i32, (kv.batch,)),
        _ptr(k_new, "k_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _ptr(v_new, "v_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _stream(stream)))


def quest_estimate(kv: PagedKV, q, kmin, kmax, page_table, seq_lens, scores,
                   stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    _check(LIB.quest_estimate(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        _stream(stream)))


def quest_topk_pages(kv: PagedKV, scores, seq_lens, k_pages: int, sel_pages,
                     stream=None) -> None:
    _check(LIB.quest_topk_pages(
        ctypes.byref(kv),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", torch.int32, (kv.batch,)),
        int(k_pages),
        _ptr(sel_pages, "sel_pages", torch.int32,
             (kv.batch, kv.num_kv_heads, k_pages)),
        _stream(stream)))


def quest_topk_pages_ex(kv: PagedKV, scores, seq_lens, k_pages: int,
                        n_sink: int, n_local: int, sel_pages,
                        stream=None) -> None:
    _check(LIB.quest_topk_pages_ex(
        ctypes.byref(kv),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", torch.int32, (kv.batch,)),
        int(k_pages), int(n_sink), int(n_local),
        _ptr(sel_pages, "sel_pages", torch.int32,
             (kv.batch, kv.num_kv_heads, k_pages)),
        _stream(stream)))


def quest_sparse_decode_attn(kv: PagedKV, q, k_pool, v_pool, page_table,
                             seq_lens, sel_pages, k_pages: int,
                             sm_scale: float, out, workspace,
                             stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_sparse_decode_attn(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        int(k_pages), float(sm_scale),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_decode_attn(kv: PagedKV, q, k_pool, v_pool, page_table, seq_lens,
                      sm_scale: float, out, workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_decode_attn(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        float(sm_scale),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_workspace_size(kv: PagedKV, k_pages: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.quest_workspace_size(ctypes.byref(kv), int(k_pages),
                                    ctypes.byref(n)))
    return int(n.value)


def quest_sparse_decode_step(kv: PagedKV, q, k_pool, v_pool, kmin, kmax,
                             page_table, seq_lens, k_pages: int,
                             sm_scale: float, scores, sel_pages, out,
                             workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_sparse_decode_step(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        int(k_pages), float(sm_scale),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_step_workspace_size(kv: PagedKV, k_pages: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.quest_step_workspace_size(ctypes.byref(kv), int(k_pages),
                                         ctypes.byref(n)))
    return int(n.value)


def quest_topk_sparse_decode_attn(kv: PagedKV, q, k_pool, v_pool, page_table,
                                  seq_lens, scores, k_pages: int,
                                  sm_scale: float, sel_pages, out, workspace,
                                  stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_topk_sparse_decode_attn(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        int(k_pages), float(sm_scale),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_stream_read_probe(buf, sink, stream=None) -> None:
    """Diagnostic: one streaming read of the whole of `buf` (any dtype,
    16-byte multiple); `sink` is a one-element int32/uint32 device tensor."""
    t = buf.tensor if isinstance(buf, HostPool) else buf
    nbytes = t.numel() * t.element_size()
    _check(LIB.quest_stream_read_probe(_ptr(buf, "buf", host_ok=True),
                                       ctypes.c_size_t(nbytes),
                                       _ptr(sink, "sink"), _stream(stream)))


def quest_topk_sparse_decode_attn_ex(kv: PagedKV, q, k_pool, v_pool,
                                     page_table, seq_lens, scores,
                                     k_pages: int, n_sink: int, n_local: int,
                                     sm_scale: float, sel_pages, out,
                                     workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_topk_sparse_decode_attn_ex(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        int(k_pages), int(n_sink), int(n_local), float(sm_scale),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_topk_sparse_decode_attn_splits(kv: PagedKV, q, k_pool, v_pool,
                                         page_table, seq_lens, scores,
                                         k_pages: int, n_sink: int, n_local: int,
                                         sm_scale: float, sel_pages, out,
                                         workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_topk_sparse_decode_attn_splits(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        int(k_pages), int(n_sink), int(n_local), float(sm_scale),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_topk_sparse_decode_attn_noalloc(kv: PagedKV, q, k_pool, v_pool,
                                          page_table, seq_lens, scores,
                                          k_pages: int, n_sink: int, n_local: int,
                                          sm_scale: float, sel_pages, out,
                                          stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    _check(LIB.quest_topk_sparse_decode_attn_noalloc(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        int(k_pages), int(n_sink), int(n_local), float(sm_scale),
        _ptr(sel_pages, "sel_pages", i32, (kv.batch, kv.num_kv_heads, k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _stream(stream)))


def quest_merge_attn_splits(kv: PagedKV, k_pages: int, workspace, out,
                            stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_merge_attn_splits(
        ctypes.byref(kv), int(k_pages), _ptr(workspace, "workspace"),
        ctypes.c_size_t(ws_bytes),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _stream(stream)))


def quest_estimate_heads(kv: PagedKV, q, kmin, kmax, page_table, seq_lens,
                         scores, stream=None) -> None:
    dt = kv.torch_dtype
    _check(LIB.quest_estimate_heads(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", torch.int32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", torch.int32, (kv.batch,)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_q_heads, kv.max_pages_per_seq)),
        _stream(stream)))


# Longest union list (G * k_pages) quest_union_sparse_decode_attn builds.
UNION_LIST_MAX = 4096


def quest_union_sparse_decode_attn(kv: PagedKV, q, k_pool, v_pool, page_table,
                                   seq_lens, sel_heads, k_pages: int, sm_scale: float,
                                   sel_union, out, workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    G = kv.num_q_heads // kv.num_kv_heads
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_union_sparse_decode_attn(
        ctypes.byref(kv),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(sel_heads, "sel_heads", i32, (kv.batch, kv.num_q_heads, k_pages)),
        int(k_pages), float(sm_scale),
        _ptr(sel_union, "sel_union", i32, (kv.batch, kv.num_kv_heads, G * k_pages)),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_union_pages(kv: PagedKV, sel_heads, k_pages: int, sel_union,
                      stream=None) -> None:
    G = kv.num_q_heads // kv.num_kv_heads
    _check(LIB.quest_union_pages(
        ctypes.byref(kv),
        _ptr(sel_heads, "sel_heads", torch.int32,
             (kv.batch, kv.num_q_heads, k_pages)),
        int(k_pages),
        _ptr(sel_union, "sel_union", torch.int32,
             (kv.batch, kv.num_kv_heads, G * k_pages)),
        _stream(stream)))


def quest_append_decode_attn(kv: PagedKV, k_pool, v_pool, kmin, kmax, page_table,
                             seq_lens, k_new, v_new, q, sm_scale: float, out,
                             workspace, stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.quest_append_decode_attn(
        ctypes.byref(kv),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(k_new, "k_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _ptr(v_new, "v_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        float(sm_scale),
        _ptr(out, "out", torch.float32, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(workspace, "workspace"), ctypes.c_size_t(ws_bytes),
        _stream(stream)))


def quest_append_estimate(kv: PagedKV, k_pool, v_pool, kmin, kmax, page_table,
                          seq_lens, k_new, v_new, q, scores,
                          stream=None) -> None:
    dt = kv.torch_dtype
    i32 = torch.int32
    _check(LIB.quest_append_estimate(
        ctypes.byref(kv),
        _ptr(k_pool, "k_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(v_pool, "v_pool", dt, _pool_shape(kv), host_ok=True),
        _ptr(kmin, "kmin", dt, _meta_shape(kv)),
        _ptr(kmax, "kmax", dt, _meta_shape(kv)),
        _ptr(page_table, "page_table", i32, (kv.batch, kv.max_pages_per_seq)),
        _ptr(seq_lens, "seq_lens", i32, (kv.batch,)),
        _ptr(k_new, "k_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _ptr(v_new, "v_new", dt, (kv.batch, kv.num_kv_heads, kv.head_dim)),
        _ptr(q, "q", dt, (kv.batch, kv.num_q_heads, kv.head_dim)),
        _ptr(scores, "scores", torch.float32,
             (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)),
        _stream(stream)))
