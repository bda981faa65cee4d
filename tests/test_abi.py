"""The C ABI on the host: libquest.so loads, exports every symbol
include/quest.h declares, and rejects bad arguments with the documented
status before any HIP call (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import query_aware_kv_amd as qa
from query_aware_kv_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quest.h")

FAKE = 1 << 20  # an aligned non-null address; never dereferenced here


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"QUEST_API\s+[\w\s\*]+?\b(quest_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert set(names) >= {"quest_update_page_meta", "quest_estimate",
                          "quest_topk_pages", "quest_sparse_decode_attn",
                          "quest_decode_attn", "quest_workspace_size",
                          "quest_status_string", "quest_last_error"}
    lib = ctypes.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def kv(**kw):
    base = dict(batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128,
                page_size=16, num_pool_pages=2048, max_pages_per_seq=2048,
                dtype=_abi.QUEST_F16)
    base.update(kw)
    return _abi.PagedKV(**base)


def ws_size(k, pages=128):
    n = ctypes.c_size_t(0)
    st = qa.LIB.quest_workspace_size(ctypes.byref(k), pages, ctypes.byref(n))
    return st, n.value


def test_status_strings():
    assert qa.LIB.quest_status_string(0) == b"ok"
    assert b"workspace" in qa.LIB.quest_status_string(3)
    assert qa.LIB.quest_status_string(99) == b"unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, _abi.QUEST_ERR_UNSUPPORTED),
    ("page_size", 64, _abi.QUEST_ERR_UNSUPPORTED),
    ("page_size", 8, _abi.QUEST_ERR_UNSUPPORTED),
    ("dtype", 7, _abi.QUEST_ERR_UNSUPPORTED),
    ("num_kv_heads", 5, _abi.QUEST_ERR_INVALID_ARGUMENT),   # 32 % 5 != 0
    ("num_q_heads", 96, _abi.QUEST_ERR_UNSUPPORTED),        # G = 3
    ("batch", 0, _abi.QUEST_ERR_INVALID_ARGUMENT),
    ("max_pages_per_seq", 0, _abi.QUEST_ERR_INVALID_ARGUMENT),
    ("batch", 2048, _abi.QUEST_ERR_UNSUPPORTED),            # 65536 rows > 65535
])
def test_geometry_validation(field, value, status):
    st, _ = ws_size(kv(**{field: value}))
    assert st == status
    assert qa.LIB.quest_last_error().decode()


def test_null_kv_and_null_out_param():
    n = ctypes.c_size_t(0)
    assert qa.LIB.quest_workspace_size(None, 8, ctypes.byref(n)) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    k = kv()
    assert qa.LIB.quest_workspace_size(ctypes.byref(k), 8, None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_workspace_size(ctypes.byref(k), 0, ctypes.byref(n)) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT


def test_workspace_size_grows_with_pages_and_zero_when_unsplit():
    st, small = ws_size(kv(), 128)
    assert st == 0 and small > 0
    st, big = ws_size(kv(), 2048)
    assert st == 0 and big > small
    # 4 pages fit one workgroup: no split, no workspace
    st, none = ws_size(kv(num_q_heads=1, num_kv_heads=1), 4)
    assert st == 0 and none == 0


def test_estimate_rejects_null_and_misaligned():
    k = kv()
    P = ctypes.c_void_p
    args = [P(FAKE)] * 6
    for i, name in enumerate(["q", "kmin", "kmax", "page_table", "seq_lens",
                              "scores"]):
        bad = list(args)
        bad[i] = None
        st = qa.LIB.quest_estimate(ctypes.byref(k), *bad, None)
        assert st == _abi.QUEST_ERR_INVALID_ARGUMENT
        assert name in qa.LIB.quest_last_error().decode()
    bad = list(args)
    bad[0] = P(FAKE + 8)                     # q must be 16-byte aligned
    assert qa.LIB.quest_estimate(ctypes.byref(k), *bad, None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    assert "misaligned" in qa.LIB.quest_last_error().decode()


def test_topk_validation():
    k = kv()
    P = ctypes.c_void_p
    assert qa.LIB.quest_topk_pages(ctypes.byref(k), P(FAKE), P(FAKE), 0,
                                   P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    big = kv(max_pages_per_seq=40000)
    assert qa.LIB.quest_topk_pages(ctypes.byref(big), P(FAKE), P(FAKE), 8,
                                   P(FAKE), None) == _abi.QUEST_ERR_UNSUPPORTED


def test_attention_workspace_and_scale_checks():
    k = kv()
    P = ctypes.c_void_p
    st, need = ws_size(k, 128)
    common = [P(FAKE)] * 6                 # q, k_pool, v_pool, pt, lens, sel
    st = qa.LIB.quest_sparse_decode_attn(ctypes.byref(k), *common, 128, 0.088,
                                         P(FAKE), P(FAKE), need - 1, None)
    assert st == _abi.QUEST_ERR_WORKSPACE_TOO_SMALL
    st = qa.LIB.quest_sparse_decode_attn(ctypes.byref(k), *common, 128, 0.088,
                                         P(FAKE), None, need, None)
    assert st == _abi.QUEST_ERR_WORKSPACE_TOO_SMALL
    st = qa.LIB.quest_sparse_decode_attn(ctypes.byref(k), *common, 128,
                                         float("nan"), P(FAKE), P(FAKE), need,
                                         None)
    assert st == _abi.QUEST_ERR_INVALID_ARGUMENT
    st = qa.LIB.quest_sparse_decode_attn(ctypes.byref(k), *common, 0, 0.088,
                                         P(FAKE), P(FAKE), need, None)
    assert st == _abi.QUEST_ERR_INVALID_ARGUMENT
    st, dneed = ws_size(k, k.max_pages_per_seq)
    st = qa.LIB.quest_decode_attn(ctypes.byref(k), *common[:5], 0.088,
                                  P(FAKE), P(FAKE), dneed - 16, None)
    assert st == _abi.QUEST_ERR_WORKSPACE_TOO_SMALL


def test_meta_mode_validation():
    k = kv()
    P = ctypes.c_void_p
    f = qa.LIB.quest_update_page_meta
    # k_new without v_new
    assert f(ctypes.byref(k), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
             P(FAKE), None, P(FAKE), None, None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    # append mode with first_token
    assert f(ctypes.byref(k), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
             P(FAKE), P(FAKE), P(FAKE), P(FAKE), None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    # append mode needs v_pool
    assert f(ctypes.byref(k), P(FAKE), None, P(FAKE), P(FAKE), P(FAKE),
             P(FAKE), None, P(FAKE), P(FAKE), None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    # rebuild mode with a null kmin
    assert f(ctypes.byref(k), P(FAKE), None, None, P(FAKE), P(FAKE), P(FAKE),
             None, None, None, None) == _abi.QUEST_ERR_INVALID_ARGUMENT


def test_python_binding_rejects_host_tensors():
    import torch
    k = qa.paged_kv(1, 1, 1, 4, 4, torch.float16)
    t = torch.zeros(1, 1, 128, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        qa.quest_estimate(k, t, t, t, t, t, t)


def test_fused_step_is_switched_off():
    """The one-launch step is switched off: it refuses work before any launch."""
    k = kv()
    P = ctypes.c_void_p
    st = qa.LIB.quest_sparse_decode_step(
        ctypes.byref(k), *([P(FAKE)] * 7), 128, 0.088, P(FAKE), P(FAKE),
        P(FAKE), P(FAKE), 1 << 30, None)
    assert st == _abi.QUEST_ERR_UNSUPPORTED
    assert "switched off" in qa.LIB.quest_last_error().decode()


def test_stream_read_probe_validation():
    P = ctypes.c_void_p
    f = qa.LIB.quest_stream_read_probe
    assert f(None, 1024, P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 1024, None, None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert f(P(FAKE + 8), 1024, P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert f(P(FAKE), 1000, P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert "multiple of 16" in qa.LIB.quest_last_error().decode()
    assert f(P(FAKE), 0, P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT


def test_topk_ex_forced_count_validation():
    k = kv()
    P = ctypes.c_void_p
    f = qa.LIB.quest_topk_pages_ex
    for ns, nl in ((-1, 0), (0, -1), (5, 4), (8, 1)):
        assert f(ctypes.byref(k), P(FAKE), P(FAKE), 8, ns, nl, P(FAKE), None) == \
            _abi.QUEST_ERR_INVALID_ARGUMENT
        assert "n_sink" in qa.LIB.quest_last_error().decode()
    st, need = ws_size(k, 8)
    common = [P(FAKE)] * 6                 # q, k_pool, v_pool, pt, lens, scores
    assert qa.LIB.quest_topk_sparse_decode_attn_ex(
        ctypes.byref(k), *common, 8, 6, 3, 0.088, P(FAKE), P(FAKE), P(FAKE),
        need, None) == _abi.QUEST_ERR_INVALID_ARGUMENT


def test_plain_calls_name_themselves_in_errors():
    k = kv()
    P = ctypes.c_void_p
    assert qa.LIB.quest_topk_pages(ctypes.byref(k), P(FAKE), P(FAKE), 0,
                                   P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_last_error().decode().startswith("quest_topk_pages:")


def test_union_and_heads_validation():
    k = kv(num_q_heads=32, num_kv_heads=8)
    P = ctypes.c_void_p
    assert qa.LIB.quest_union_pages(ctypes.byref(k), P(FAKE), 0, P(FAKE), None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_union_pages(ctypes.byref(k), None, 8, P(FAKE), None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    big = kv(max_pages_per_seq=40000)
    assert qa.LIB.quest_union_pages(ctypes.byref(big), P(FAKE), 8, P(FAKE), None) == \
        _abi.QUEST_ERR_UNSUPPORTED
    assert qa.LIB.quest_estimate_heads(ctypes.byref(k), *([P(FAKE)] * 5), None,
                                       None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert "scores" in qa.LIB.quest_last_error().decode()


def test_host_device_pointer_rejects_null():
    P = ctypes.c_void_p
    out = ctypes.c_void_p()
    assert qa.LIB.quest_host_device_pointer(None, ctypes.byref(out)) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_host_device_pointer(P(FAKE), None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT


def test_host_pool_needs_pinned_cpu_tensor():
    import torch
    with pytest.raises(ValueError, match="pinned"):
        qa.HostPool(torch.zeros(4, 128, dtype=torch.float16))


def test_append_estimate_validation():
    k = kv()
    P = ctypes.c_void_p
    args = [P(FAKE)] * 10   # k_pool v_pool kmin kmax pt lens k_new v_new q scores
    for i, name in enumerate(["k_pool", "v_pool", "kmin", "kmax", "page_table",
                              "seq_lens", "k_new", "v_new", "q", "scores"]):
        bad = list(args)
        bad[i] = None
        assert qa.LIB.quest_append_estimate(ctypes.byref(k), *bad, None) == \
            _abi.QUEST_ERR_INVALID_ARGUMENT
        assert name in qa.LIB.quest_last_error().decode()


def test_append_decode_attn_validation():
    k = kv()
    P = ctypes.c_void_p
    st, need = ws_size(k, k.max_pages_per_seq)
    names = ["k_pool", "v_pool", "kmin", "kmax", "page_table", "seq_lens", "k_new",
             "v_new", "q"]
    args = [P(FAKE)] * len(names)
    for i, name in enumerate(names):
        bad = list(args)
        bad[i] = None
        assert qa.LIB.quest_append_decode_attn(ctypes.byref(k), *bad, 0.088, P(FAKE),
                                               P(FAKE), need, None) == \
            _abi.QUEST_ERR_INVALID_ARGUMENT
        assert name in qa.LIB.quest_last_error().decode()
    assert qa.LIB.quest_append_decode_attn(ctypes.byref(k), *args, 0.088, None, P(FAKE),
                                           need, None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_append_decode_attn(ctypes.byref(k), *args, float("nan"), P(FAKE),
                                           P(FAKE), need, None) == \
        _abi.QUEST_ERR_INVALID_ARGUMENT
    assert qa.LIB.quest_append_decode_attn(ctypes.byref(k), *args, 0.088, P(FAKE),
                                           P(FAKE), need - 16, None) == \
        _abi.QUEST_ERR_WORKSPACE_TOO_SMALL


def test_union_sparse_decode_attn_validation():
    k = kv(num_kv_heads=8)                          # groups of 4
    P = ctypes.c_void_p
    kp = 128
    st, need = ws_size(k, 4 * kp)
    assert st == 0 and need > 0
    names = ["q", "k_pool", "v_pool", "page_table", "seq_lens", "sel_heads"]
    args = [P(FAKE)] * len(names)
    call = qa.LIB.quest_union_sparse_decode_attn
    for i, name in enumerate(names):
        bad = list(args)
        bad[i] = None
        assert call(ctypes.byref(k), *bad, kp, 0.088, P(FAKE), P(FAKE), P(FAKE), need,
                    None) == _abi.QUEST_ERR_INVALID_ARGUMENT
        assert name in qa.LIB.quest_last_error().decode()
    for pos in range(3):                             # sel_union, out, workspace
        tail = [P(FAKE), P(FAKE), P(FAKE)]
        tail[pos] = None
        want = _abi.QUEST_ERR_WORKSPACE_TOO_SMALL if pos == 2 else \
            _abi.QUEST_ERR_INVALID_ARGUMENT
        assert call(ctypes.byref(k), *args, kp, 0.088, *tail, need, None) == want
    assert call(ctypes.byref(k), *args, 0, 0.088, P(FAKE), P(FAKE), P(FAKE), need,
                None) == _abi.QUEST_ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(k), *args, kp, 0.088, P(FAKE), P(FAKE), P(FAKE), need - 16,
                None) == _abi.QUEST_ERR_WORKSPACE_TOO_SMALL
    # the union list must fit the workgroups' LDS: G * k_pages <= 4096
    assert call(ctypes.byref(k), *args, 1025, 0.088, P(FAKE), P(FAKE), P(FAKE), 1 << 40,
                None) == _abi.QUEST_ERR_UNSUPPORTED
    assert "4096" in qa.LIB.quest_last_error().decode()
    big = kv(num_kv_heads=8, max_pages_per_seq=32769, num_pool_pages=32769)
    assert call(ctypes.byref(big), *args, kp, 0.088, P(FAKE), P(FAKE), P(FAKE), 1 << 40,
                None) == _abi.QUEST_ERR_UNSUPPORTED


def test_last_error_is_per_thread():
    """Each host thread reads the message of its own last failed call."""
    import threading
    k = kv()
    P = ctypes.c_void_p
    step = threading.Barrier(2)
    seen = {}

    def a():
        assert qa.LIB.quest_topk_pages(ctypes.byref(k), P(FAKE), P(FAKE), 0,
                                       P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
        step.wait()
        step.wait()  # b has failed in between
        seen["a"] = qa.LIB.quest_last_error().decode()

    def b():
        step.wait()
        assert qa.LIB.quest_topk_pages_ex(ctypes.byref(k), P(FAKE), P(FAKE), 8, -1, 0,
                                          P(FAKE), None) == _abi.QUEST_ERR_INVALID_ARGUMENT
        step.wait()
        seen["b"] = qa.LIB.quest_last_error().decode()

    ts = [threading.Thread(target=f) for f in (a, b)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=30)
    assert seen["a"].startswith("quest_topk_pages:") and "k_pages" in seen["a"]
    assert seen["b"].startswith("quest_topk_pages_ex:") and "n_sink" in seen["b"]


def test_paged_kv_like_reads_the_geometry_off_the_tensors():
    import torch
    q = torch.zeros(3, 8, 128, dtype=torch.bfloat16)
    k_pool = torch.zeros(10, 2, 32, 128, dtype=torch.bfloat16)
    pt = torch.zeros(3, 7, dtype=torch.int32)
    kv = qa.paged_kv_like(q, k_pool, pt)
    assert (kv.batch, kv.num_q_heads, kv.num_kv_heads, kv.num_pool_pages,
            kv.max_pages_per_seq, kv.page_size, kv.head_dim) == (3, 8, 2, 10, 7, 32, 128)
    assert kv.dtype == _abi.QUEST_BF16
    st, n = ws_size(kv, 7)
    assert st == _abi.QUEST_OK
    with pytest.raises(ValueError):
        qa.paged_kv_like(q, k_pool[..., :64], pt)      # head dims disagree
    with pytest.raises(ValueError):
        qa.paged_kv_like(q, k_pool, pt[:2])            # batch disagrees
    with pytest.raises(ValueError):
        qa.paged_kv_like(q.float(), k_pool.float(), pt)  # no float32 caches


def test_noalloc_refuses_geometries_past_its_scratch():
    """The allocation-free entry point holds 8 MiB of split scratch per GPU:
    a geometry that needs more is refused on the host, before any HIP call
    (2048 rows x 1024 kept pages: 64 MiB of partials)."""
    k = kv(batch=64, num_pool_pages=16, max_pages_per_seq=1024)
    st, need = ws_size(k, 1024)
    assert st == 0 and need > 8 << 20
    P = ctypes.c_void_p
    st = qa.LIB.quest_topk_sparse_decode_attn_noalloc(
        ctypes.byref(k), *[P(FAKE)] * 6, 1024, 0, 0, 0.088, P(FAKE), P(FAKE), None)
    assert st == _abi.QUEST_ERR_UNSUPPORTED
    msg = qa.LIB.quest_last_error().decode()
    assert "scratch" in msg and str(8 << 20) in msg
    # bad counts are still argument errors
    st = qa.LIB.quest_topk_sparse_decode_attn_noalloc(
        ctypes.byref(kv()), *[P(FAKE)] * 6, 0, 0, 0, 0.088, P(FAKE), P(FAKE), None)
    assert st == _abi.QUEST_ERR_INVALID_ARGUMENT
