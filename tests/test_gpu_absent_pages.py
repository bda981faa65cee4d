"""Page-table entries below a request's page count that name no pool page
(negative, or at or past num_pool_pages) are absent pages, as quest.h
states: their boxes are not built, their bound is -inf, attention skips
their tokens, and nothing outside the buffers is read.  Checked against
the oracle run on the same table with those entries pointed at a valid
page, whose results at the absent positions are then replaced by what
absence means (-inf bounds, no tokens)."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


@pytest.mark.parametrize("budget", [96, 50 * 16])   # k = 6; k = 50 keeps every page
@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("G", [1, 2])
def test_page_ids_outside_the_pool_are_absent(G, select, budget):
    lens = (700, 333)
    wl = C.workload(2, 4 * G, 4, lens, budget, "f16", seed=90 + G, name="absent")
    C.say(f"[case] absent page ids G={G} {select} lens={lens} k={wl.k_pages}")
    c = C.draw(wl)
    kv = c["kv"]
    P = kv.num_pool_pages
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(90 + G)
    absent = {}
    for b, L in enumerate(lens):
        n = -(-L // 16)
        js = sorted(rng.choice(n - 1, 5, replace=False).tolist())  # full pages only
        for j, v in zip(js, [-1, -7, P, P + 100, 2 ** 31 - 1]):
            pt[b, j] = v
        absent[b] = js
    c["page_table"] = torch.from_numpy(pt.astype(np.int32)).cuda()
    kmin, kmax = C.gpu_meta(c)
    step = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    out = step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
               c["seq_lens"])
    dense = qa.DenseDecode(kv, SM)
    d = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()

    o = C.oracle_inputs(c)
    ok = o["page_table"].copy()
    spare = int(pt[0, [j for j in range(-(-lens[0] // 16)) if j not in absent[0]][0]])
    for b, js in absent.items():
        ok[b, js] = spare                 # a full, valid page stands in
    omin, omax = O.page_meta(o["k_pool"], ok, o["seq_lens"], 16)
    valid_pages = sorted({int(pt[b, j]) for b, L in enumerate(lens)
                          for j in range(-(-L // 16)) if j not in absent[b]})
    C.assert_meta_bitexact(kmin, kmax, omin, omax, valid_pages)
    s_ora = O.estimate(o["q"], omin, omax, ok, o["seq_lens"], 16, kv.max_pages_per_seq)
    for b, js in absent.items():
        s_ora[b, :, js] = -np.inf
    s_gpu = step.scores.cpu().numpy().astype(np.float64)
    for b, js in absent.items():
        assert np.all(np.isneginf(s_gpu[b, :, js]))
    fin = np.isfinite(s_ora)
    err = np.abs(s_gpu[fin] - s_ora[fin])
    assert np.all(err <= C.SCORE_RTOL * np.abs(s_ora[fin]))
    sel = step.sel.cpu().numpy().astype(np.int64)
    C.assert_sets_match(sel, s_ora, o["seq_lens"], wl.k_pages)
    kept = sel.copy()
    for b, js in absent.items():
        kept[b][np.isin(kept[b], js)] = -1   # absent pages contribute no tokens
    ref = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"], ok, o["seq_lens"],
                             kept, SM, 16)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)
    every = np.full((2, kv.num_kv_heads, kv.max_pages_per_seq), -1, dtype=np.int64)
    for b, L in enumerate(lens):
        vp = [j for j in range(-(-L // 16)) if j not in absent[b]]
        every[b, :, :len(vp)] = vp
    ref_d = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"], ok, o["seq_lens"],
                               every, SM, 16)
    C.assert_attention_close(d.cpu().numpy().astype(np.float64), ref_d)


def test_lengths_past_the_table_are_clamped():
    """A length above max_pages_per_seq * page_size counts as that many
    tokens (quest.h): with a request whose pages are all full, raising its
    length past the table changes no box, bound, list or output bit."""
    lens = (64 * 16, 500)
    wl = C.workload(2, 8, 4, lens, 20 * 16, "f16", seed=95, permute=True,
                    name="clamped")
    C.say(f"[case] lengths past the table lens={lens} max_pages={wl.max_pages}")
    c = C.draw(wl)
    kv = c["kv"]
    assert kv.max_pages_per_seq == 64
    long_lens = c["seq_lens"].clone()
    long_lens[0] += 777
    res = []
    for L in (c["seq_lens"], long_lens):
        kmin, kmax = qa.alloc_meta(kv)
        kmin.fill_(float("nan"))
        kmax.fill_(float("nan"))
        qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                                  c["page_table"], L)
        step = qa.SparseDecodeStep(kv, wl.k_pages, SM)
        step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"], L)
        dense = qa.DenseDecode(kv, SM)
        d = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], L)
        torch.cuda.synchronize()
        res.append((kmin.view(torch.int16).clone(), kmax.view(torch.int16).clone(),
                    step.scores.view(torch.int32).clone(), step.sel.clone(),
                    step.out.view(torch.int32).clone(), d.view(torch.int32).clone()))
    used = torch.tensor(C.used_pages(c["page_table"].cpu().numpy(), lens), device="cuda")
    a, b = res
    assert torch.equal(a[0][used], b[0][used]) and torch.equal(a[1][used], b[1][used])
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)
