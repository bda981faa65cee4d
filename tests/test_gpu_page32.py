"""32-token pages ("Guide to Quest", Best Practices 1: B = 32 halves the
metadata and suits 128K+ contexts) through every call: metadata rebuild and
append bit for bit, bounds, Top-K, sparse (both paths), dense and union
attention against the oracle run with page_size = 32."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
S = 32
CASES = {
    # name: (B, Hq, Hkv, lens, budget, dtype, permute, outliers, planted)
    "p32_mha_ragged_f16": (3, 4, 4, (1, 45, 1000), 320, "f16", True, 4, 0),
    "p32_mha_bf16": (2, 2, 2, (33, 2047), 256, "bf16", True, 0, 0),
    "p32_gqa4_f16": (2, 16, 4, (513, 2000), 480, "f16", False, 4, 0),
    "p32_gqa8_bf16": (1, 16, 2, (1500,), 320, "bf16", True, 0, 0),
    "p32_planted_f16": (2, 8, 8, (4096, 3000), 512, "f16", False, 4, 5),
    "p32_with_empty": (3, 2, 2, (0, 33, 32), 64, "f16", True, 0, 0),
}


def make(name, seed=0):
    B, Hq, Hkv, lens, budget, dt, perm, outl, plant = CASES[name]
    wl = C.workload(B, Hq, Hkv, lens, budget, dt, seed, perm, outl, plant, name,
                    page_size=S)
    C.say(f"[case] {name} B={B} Hq={Hq} Hkv={Hkv} lens={lens} k={wl.k_pages} "
          f"{dt} page_size={S}")
    return wl, C.draw(wl)


def oracle_meta(o):
    return O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], S)


@pytest.mark.parametrize("name", sorted(CASES))
def test_meta_rebuild_bitexact_p32(name):
    wl, c = make(name)
    kmin, kmax = C.gpu_meta(c)
    o = C.oracle_inputs(c)
    omin, omax = oracle_meta(o)
    C.assert_meta_bitexact(kmin, kmax, omin, omax,
                           C.used_pages(o["page_table"], o["seq_lens"], S))


@pytest.mark.parametrize("name", ["p32_mha_ragged_f16", "p32_gqa4_f16"])
def test_meta_append_p32(name):
    """The last 40 tokens appended one at a time (crossing page boundaries)
    give the full rebuild's boxes and write the pool rows bit for bit."""
    wl, c = make(name)
    kv = c["kv"]
    full = c["seq_lens"].clone()
    start = torch.clamp(full - 40, min=0)
    o = C.oracle_inputs(c)
    omin, omax = oracle_meta(o)
    pages = C.used_pages(o["page_table"], o["seq_lens"], S)
    pt = c["page_table"].long()
    kp, vp = c["k_pool"].clone(), c["v_pool"].clone()
    B = kv.batch
    news = []
    for s in range(40):
        pos = start + s
        k_new = torch.zeros(B, kv.num_kv_heads, 128, dtype=kp.dtype, device="cuda")
        v_new = torch.zeros_like(k_new)
        active = pos < full
        for b in range(B):
            if active[b]:
                p = pt[b, pos[b] // S]
                k_new[b] = kp[p, :, pos[b] % S]
                v_new[b] = vp[p, :, pos[b] % S]
        news.append((k_new, v_new, active))
    for b in range(B):
        for x in range(int(start[b]), int(full[b])):
            kp[pt[b, x // S], :, x % S] = float("nan")
            vp[pt[b, x // S], :, x % S] = float("nan")
    amin, amax = qa.alloc_meta(kv)
    amin.fill_(float("nan"))
    amax.fill_(float("nan"))
    qa.quest_update_page_meta(kv, kp, vp, amin, amax, c["page_table"], start.cuda())
    lens = start.clone()
    for k_new, v_new, active in news:
        lens = lens + active.to(torch.int32)
        L = torch.where(active, lens, torch.zeros_like(lens)).to(torch.int32)
        qa.quest_update_page_meta(kv, kp, vp, amin, amax, c["page_table"], L.cuda(),
                                  k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    C.assert_meta_bitexact(amin, amax, omin, omax, pages)
    for b in range(B):
        for x in range(int(full[b])):
            p = pt[b, x // S]
            assert torch.equal(kp[p, :, x % S].view(torch.int16),
                               c["k_pool"][p, :, x % S].view(torch.int16))


@pytest.mark.parametrize("name", sorted(CASES))
def test_estimate_p32(name):
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), 5.0,
                   device="cuda")
    qa.quest_estimate(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], s)
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    omin, omax = oracle_meta(o)
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], S,
                       kv.max_pages_per_seq)
    C.assert_scores_close(s.cpu().numpy().astype(np.float64), s_ora, o["seq_lens"], S)


def test_topk_p32_rows_follow_page_count():
    """Top-K counts pages as ceil(L / 32)."""
    rows, mp, k = 6, 512, 40
    g = np.random.default_rng(5)
    lens_tok = [0, 1, 32, 33, 40 * 32, mp * 32 - 7]
    s = g.integers(-5, 6, (rows, 1, mp)).astype(np.float32)
    kv = qa.paged_kv(rows, 1, 1, 1, mp, torch.float16, page_size=S)
    sel = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    qa.quest_topk_pages(kv, torch.from_numpy(s).cuda(),
                        torch.tensor(lens_tok, dtype=torch.int32, device="cuda"), k, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for r, L in enumerate(lens_tok):
        n = -(-L // S)
        assert np.array_equal(got[r, 0], O.topk_pages(s[r, 0].astype(np.float64), n, k))


@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_step_p32(name, select):
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s_gpu, sel_gpu, out_gpu = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM,
                                             select=select)
    o = C.oracle_inputs(c)
    omin, omax = oracle_meta(o)
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], S,
                       kv.max_pages_per_seq)
    C.assert_scores_close(s_gpu, s_ora, o["seq_lens"], S)
    C.assert_sets_match(sel_gpu, s_ora, o["seq_lens"], wl.k_pages, S)
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"], sel_gpu, SM, S)
    C.assert_attention_close(out_gpu, out_ora)


@pytest.mark.parametrize("name", sorted(CASES))
def test_dense_p32(name):
    wl, c = make(name)
    out = qa.DenseDecode(c["kv"], SM)(c["q"], c["k_pool"], c["v_pool"],
                                      c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    ref = O.dense_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                            o["seq_lens"], SM, S)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("name", ["p32_gqa4_f16", "p32_gqa8_bf16"])
def test_union_step_p32(name):
    wl, c = make(name)
    kv = c["kv"]
    G = kv.num_q_heads // kv.num_kv_heads
    kmin, kmax = C.gpu_meta(c)
    st = qa.UnionDecodeStep(kv, wl.k_pages, SM)
    out = st(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
             c["seq_lens"])
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    omin, omax = oracle_meta(o)
    s_ora = O.estimate_heads(o["q"], omin, omax, o["page_table"], o["seq_lens"], S,
                             kv.max_pages_per_seq)
    sel_heads = st.sel_heads.cpu().numpy().astype(np.int64)
    C.assert_sets_match(sel_heads, s_ora, o["seq_lens"], wl.k_pages, S)
    sel = st.sel.cpu().numpy().astype(np.int64)
    assert np.array_equal(sel, O.union_pages(sel_heads, G))
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"], sel, SM, S)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), out_ora)
