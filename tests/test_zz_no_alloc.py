"""The allocation-free entry point (quest_topk_sparse_decode_attn_noalloc):
its split partials live in the library's per-GPU scratch array instead of a
caller workspace.  Through the C ABI, two calls in a row -- a full-size
LongChat layer, then a smaller ragged batch, so the second call runs over
the first one's leftover partials -- each give the selection and the output
of quest_topk_sparse_decode_attn_ex bit for bit, and a geometry whose
partials exceed the scratch is refused before any launch."""
import math

import pytest
import torch

import query_aware_kv_amd as qa
import synth

import gpu_cases as C
from test_gpu_parity import make

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


def _compare(c, k, n_sink=0, n_local=0):
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    ref = qa.SparseDecodeStep(kv, k, SM, select="attention", n_sink=n_sink,
                              n_local=n_local)
    ref(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"], c["seq_lens"])
    sel = torch.full_like(ref.sel, -777)
    out = torch.full_like(ref.out, float("nan"))
    qa.quest_topk_sparse_decode_attn_noalloc(
        kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"],
        ref.scores, k, n_sink, n_local, SM, sel, out)
    torch.cuda.synchronize()
    assert torch.equal(sel, ref.sel)
    assert torch.equal(out.view(torch.int32), ref.out.view(torch.int32))


def test_noalloc_matches_workspace_entry_point_twice():
    wl = synth.longchat_layer_workload()
    C.say(f"[case] noalloc 1/2: {wl.name} (32 heads, 32K, k={wl.k_pages})")
    c = synth.draw_layer(wl, 0, "cuda")
    c["kv"] = qa.paged_kv(1, 32, 32, wl.pool_pages(), wl.max_pages, wl.torch_dtype)
    _compare(c, wl.k_pages)
    del c
    C.say("[case] noalloc 2/2: mha_ragged_f16 (smaller), with forced pages")
    wl2, c2 = make("mha_ragged_f16")
    _compare(c2, wl2.k_pages, n_sink=1, n_local=2)


def test_noalloc_refuses_oversize_scratch():
    # 2048 (request, kv-head) rows x 1024 kept pages: 64 MiB of partials;
    # a 16-page pool keeps the tensors small (the call is refused before
    # any launch, so nothing is read)
    d = "cuda"
    q = torch.zeros(64, 32, 128, dtype=torch.float16, device=d)
    pool = torch.zeros(16, 32, 16, 128, dtype=torch.float16, device=d)
    kvs = qa.paged_kv(64, 32, 32, 16, 1024, torch.float16)
    need_s = qa.quest_workspace_size(kvs, 1024)
    assert need_s > 8 << 20
    with pytest.raises(qa.QuestError) as e:
        qa.quest_topk_sparse_decode_attn_noalloc(
            kvs, q, pool, pool,
            torch.zeros(64, 1024, dtype=torch.int32, device=d),
            torch.zeros(64, dtype=torch.int32, device=d),
            torch.zeros(64, 32, 1024, dtype=torch.float32, device=d), 1024, 0, 0, SM,
            torch.zeros(64, 32, 1024, dtype=torch.int32, device=d),
            torch.zeros(64, 32, 128, dtype=torch.float32, device=d))
    assert e.value.status == qa.QUEST_ERR_UNSUPPORTED
    assert "scratch" in str(e.value)
