"""Forced sink and local-window pages ("Guide to Quest" §3 and
Implementation Step 2) on the GPU: quest_topk_pages_ex bit for bit against
the oracle's topk_pages_forced, the one-launch Top-K + attention variant
against the two separate calls, and a whole step against the oracle."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C
from test_gpu_parity import _topk_case, make

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


@pytest.mark.parametrize("mp,k,ns,nl", [
    (64, 8, 2, 2), (64, 8, 4, 4), (1024, 100, 4, 16), (1027, 100, 3, 5),
    (2048, 128, 2, 2),
    (2048, 128, 64, 64), (2048, 128, 0, 127), (4100, 256, 1, 0),
    (8192, 512, 0, 32), (32768, 4096, 16, 16)])
def test_topk_ex_bitexact(mp, k, ns, nl):
    rows = 16
    g = np.random.default_rng(7 * mp + k + ns)
    n_list = [mp, k, k + 1, k + 2, max(1, k - 1), 0, 1, ns + nl + 1] + \
        [int(x) for x in g.integers(1, mp + 1, rows - 8)]
    n_list = [min(n, mp) for n in n_list]
    C.say(f"[case] topk_ex mp={mp} k={k} sink={ns} local={nl} n={n_list}")
    s = _topk_case(rows, n_list, mp, k, seed=mp + 1)
    for r, n in enumerate(n_list):           # forced pages' scores are never used
        if n > k:
            s[r, 0, :ns] = np.nan
            s[r, 0, n - nl:n] = np.nan
    lens = torch.tensor([n * 16 for n in n_list], dtype=torch.int32)
    kv = qa.paged_kv(rows, 1, 1, 1, mp, torch.float16)
    sel = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    qa.quest_topk_pages_ex(kv, torch.from_numpy(s).cuda(), lens.cuda(), k, ns, nl, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for r in range(rows):
        ref = O.topk_pages_forced(s[r, 0].astype(np.float64), n_list[r], k, ns, nl)
        assert np.array_equal(got[r, 0], ref), f"row {r} n={n_list[r]}"


def test_topk_ex_zero_forced_is_plain():
    mp, k, rows = 2048, 128, 8
    n_list = [2048, 129, 128, 1000, 5, 0, 300, 2047]
    s = _topk_case(rows, n_list, mp, k, seed=11)
    lens = torch.tensor([n * 16 for n in n_list], dtype=torch.int32, device="cuda")
    kv = qa.paged_kv(rows, 1, 1, 1, mp, torch.float16)
    a = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    b = torch.full((rows, 1, k), -9, dtype=torch.int32, device="cuda")
    sc = torch.from_numpy(s).cuda()
    qa.quest_topk_pages_ex(kv, sc, lens, k, 0, 0, a)
    qa.quest_topk_pages(kv, sc, lens, k, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,ns,nl", [
    ("mha_ragged_f16", 1, 2), ("gqa4_f16", 2, 2), ("gqa8_f16", 0, 4),
    ("planted_f16", 4, 0), ("with_empty_request", 1, 1), ("tiny_ref", 4, 4)])
def test_topk_attn_ex_equals_separate_calls(name, ns, nl):
    wl, c = make(name)
    kv = c["kv"]
    k = wl.k_pages
    kmin, kmax = C.gpu_meta(c)
    a = qa.SparseDecodeStep(kv, k, SM, select="attention", n_sink=ns, n_local=nl)
    b = qa.SparseDecodeStep(kv, k, SM, select="separate", n_sink=ns, n_local=nl)
    a.sel.fill_(-777)
    args = (c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
            c["seq_lens"])
    a(*args)
    b(*args)
    torch.cuda.synchronize()
    assert int((a.sel == -777).sum()) == 0
    assert torch.equal(a.sel, b.sel)
    C.assert_same_up_to_split_order(a.out, b.out)


@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("name,ns,nl", [
    ("planted_f16", 1, 2), ("gqa4_f16", 2, 4), ("mha_ragged_bf16", 3, 1)])
def test_forced_step_matches_oracle(name, ns, nl, select):
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s_gpu, sel_gpu, out_gpu = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM,
                                             select=select, n_sink=ns,
                                             n_local=nl)
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                       kv.max_pages_per_seq)
    C.assert_scores_close(s_gpu, s_ora, o["seq_lens"])
    C.assert_sets_match(sel_gpu, s_ora, o["seq_lens"], wl.k_pages, n_sink=ns,
                        n_local=nl)
    for b in range(kv.batch):                       # forced pages are present
        n = -(-int(o["seq_lens"][b]) // 16)
        if n > wl.k_pages:
            want = set(range(ns)) | set(range(n - nl, n))
            for g in range(kv.num_kv_heads):
                assert want <= set(int(x) for x in sel_gpu[b, g])
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"], sel_gpu, SM, 16)
    C.assert_attention_close(out_gpu, out_ora)
