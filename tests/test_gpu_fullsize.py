"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle recomputes sampled (request, kv-head) units one
by one from host copies of the same inputs; every unit is also checked for
properties that hold at any size (valid ascending selections, planted pages
kept)."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
import synth
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


def build(wl, layer=0):
    c = synth.draw_layer(wl, layer, "cuda")
    c["kv"] = qa.paged_kv(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                          wl.pool_pages(), wl.max_pages, wl.torch_dtype,
                          page_size=wl.page_size)
    return c


def unit_oracle(c, b, heads, k, G, S=16):
    """Oracle decode step for request b restricted to kv-heads `heads`."""
    kv = c["kv"]
    pt = c["page_table"][b:b + 1].cpu().numpy().astype(np.int64)
    lens = c["seq_lens"][b:b + 1].cpu().numpy().astype(np.int64)
    n = -(-int(lens[0]) // S)
    pages = torch.from_numpy(pt[0, :n]).long().cuda()
    # compact pool: only this request's pages, only the sampled heads
    kp = C.to64(c["k_pool"][pages][:, heads])
    vp = C.to64(c["v_pool"][pages][:, heads])
    qh = [g * G + r for g in heads for r in range(G)]
    q = C.to64(c["q"][b:b + 1, qh])
    pt_c = np.zeros((1, kv.max_pages_per_seq), dtype=np.int64)
    pt_c[0, :n] = np.arange(n)
    kmin, kmax = O.page_meta(kp, pt_c, lens, S)
    s = O.estimate(q, kmin, kmax, pt_c, lens, S, kv.max_pages_per_seq)
    return dict(q=q, kp=kp, vp=vp, pt=pt_c, lens=lens, kmin=kmin, kmax=kmax,
                s=s, n=n, pages=pages)


def check_units(c, step, units, k, G, check_meta=None, S=16):
    sel_all = step.sel.cpu().numpy().astype(np.int64)
    scores = step.scores.cpu().numpy().astype(np.float64)
    out = step.out.cpu().numpy().astype(np.float64)
    kv = c["kv"]
    # properties of every row
    for b, L in enumerate(c["seq_lens"].tolist()):
        n = -(-L // S)
        for g in range(kv.num_kv_heads):
            C.assert_valid_selection(sel_all[b, g], n, k)
    worst = 0.0
    for b, heads in units:
        u = unit_oracle(c, b, heads, k, G, S)
        if check_meta is not None:
            kmin_g, kmax_g = check_meta
            gm = kmin_g[u["pages"]][:, heads].cpu().view(torch.int16)
            om = torch.from_numpy(u["kmin"]).to(kmin_g.dtype).view(torch.int16)
            assert torch.equal(gm, om), f"kmin differs (b={b})"
            gm = kmax_g[u["pages"]][:, heads].cpu().view(torch.int16)
            om = torch.from_numpy(u["kmax"]).to(kmax_g.dtype).view(torch.int16)
            assert torch.equal(gm, om), f"kmax differs (b={b})"
        s_gpu = scores[b:b + 1, heads]
        C.assert_scores_close(s_gpu, u["s"], u["lens"], S)
        sel = sel_all[b:b + 1, heads]
        C.assert_sets_match(sel, u["s"], u["lens"], k, S)
        ref = O.sparse_attention(u["q"], u["kp"], u["vp"], u["pt"], u["lens"],
                                 sel, SM, S)
        qh = [g * G + r for g in heads for r in range(G)]
        worst = max(worst, C.assert_attention_close(out[b:b + 1, qh], ref))
    return worst


def run_paths(c, k):
    """The separate-call step (the one-launch step is switched off)."""
    kmin, kmax = C.gpu_meta(c)
    sep = qa.SparseDecodeStep(c["kv"], k, SM)
    sep(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
        c["seq_lens"])
    torch.cuda.synchronize()
    return sep, (kmin, kmax)


def test_longchat_layer_32k_budget_2048():
    wl = synth.longchat_layer_workload()
    C.say(f"[case] {wl.name}: 32 heads, ctx 32768, k={wl.k_pages}")
    c = build(wl)
    step, meta = run_paths(c, wl.k_pages)
    worst = check_units(c, step, [(0, [0, 7]), (0, [19, 31])], wl.k_pages, 1,
                        check_meta=meta)
    C.say(f"  sampled attention max err {worst:.2e}")
    sel = step.sel.cpu().numpy()
    for g in range(32):   # the planted pages are kept in every head
        plant = set(synth.planted_pages(wl, 0, 0, g, 2048).tolist())
        assert plant <= set(sel[0, g].tolist()), g


def test_longchat_dense_32k_against_oracle():
    """The in-library dense baseline at the headline's size and in the
    benchmark's launch configuration (quest_decode_attn on the LongChat
    layer: one query head per kv-head, fp16, 32K tokens, 32 workgroups per
    head each walking 64 pages in chunks of 8, merged in one launch)
    against the oracle's textbook attention over every token of sampled
    heads."""
    wl = synth.longchat_layer_workload()
    C.say(f"[case] dense {wl.name}: 32 heads, ctx 32768")
    c = build(wl)
    kv = c["kv"]
    out = qa.DenseDecode(kv, SM)(c["q"], c["k_pool"], c["v_pool"],
                                 c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    heads = [3, 28]
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    lens = c["seq_lens"].cpu().numpy().astype(np.int64)
    ref = O.dense_attention(C.to64(c["q"][:, heads]), C.to64(c["k_pool"][:, heads]),
                            C.to64(c["v_pool"][:, heads]), pt, lens, SM, 16)
    worst = C.assert_attention_close(got[:, heads], ref)
    C.say(f"  dense attention max err {worst:.2e}")


@pytest.mark.parametrize("ctx,budget", [(4096, 4096), (16384, 256),
                                        (65536, 1024), (131072, 4096)])
def test_sweep_point(ctx, budget):
    wl = synth.sweep_workload(ctx, budget)
    C.say(f"[case] {wl.name}")
    c = build(wl)
    step, meta = run_paths(c, wl.k_pages)
    check_units(c, step, [(0, [5]), (0, [26])], wl.k_pages, 1, check_meta=meta)
    if wl.k_pages >= wl.max_pages:  # every page kept: the step is dense
        dense = qa.DenseDecode(c["kv"], SM)
        d = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
        torch.cuda.synchronize()
        assert (step.out - d).abs().max().item() <= 1e-5


def test_ragged_batch_bf16():
    wl = synth.ragged_batch_workload()
    C.say(f"[case] {wl.name}: lens {min(wl.seq_lens)}..{max(wl.seq_lens)} bf16")
    c = build(wl)
    step, meta = run_paths(c, wl.k_pages)
    check_units(c, step, [(0, [0]), (9, [13]), (17, [31]), (31, [2])],
                wl.k_pages, 1, check_meta=meta)


def test_gqa8_bf16_layer_32k():
    """A 32 / 4-head GQA layer (groups of 8 query heads on the matrix cores)
    in bf16 at 32K with a 2048-token budget, in the benchmark's launch
    configuration (Top-K inside the attention launch)."""
    wl = synth.Workload("gqa8_bf16_32k", 1, 32, 4, (32768,), 2048, "bf16",
                        outliers=4, base_seed=71)
    C.say(f"[case] {wl.name}: Hq 32 / Hkv 4, ctx 32768, k={wl.k_pages}, bf16")
    c = build(wl)
    step, meta = run_paths(c, wl.k_pages)
    assert step.select == "attention"
    worst = check_units(c, step, [(0, [0]), (0, [3])], wl.k_pages, wl.group,
                        check_meta=meta)
    C.say(f"  sampled attention max err {worst:.2e}")


@pytest.mark.parametrize("S", [16, 32])
def test_gqa_dense_layer_many_splits(S):
    """The dense call on a GQA layer of the multi-step workload's final size
    (32 / 8 heads, 32896 tokens: 2056 16-token or 1028 32-token pages): as
    many workgroups as the GPU holds at once (96 or 64 per kv-head at this
    kernel's occupancy), uneven page ranges, merged by the wide merge (more
    than 32 splits), against the oracle on sampled heads."""
    wl = synth.Workload(f"gqa_dense_{S}", 1, 32, 8, (32896,), 2048, "f16",
                        page_size=S, outliers=4, base_seed=73)
    C.say(f"[case] {wl.name}: Hq 32 / Hkv 8, ctx 32896, {S}-token pages, dense")
    c = build(wl)
    out = qa.DenseDecode(c["kv"], SM)(c["q"], c["k_pool"], c["v_pool"],
                                      c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    heads = [2, 7]
    qh = [g * 4 + r for g in heads for r in range(4)]
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    lens = c["seq_lens"].cpu().numpy().astype(np.int64)
    ref = O.dense_attention(C.to64(c["q"][:, qh]), C.to64(c["k_pool"][:, heads]),
                            C.to64(c["v_pool"][:, heads]), pt, lens, SM, S)
    worst = C.assert_attention_close(out.cpu().numpy().astype(np.float64)[:, qh], ref)
    C.say(f"  dense attention max err {worst:.2e}")


def test_union_layer_32k_against_oracle():
    """The union rule ("Guide to Quest", Best Practices 2) on the bench's
    GQA layer (32 / 8 heads, 32K, 2048-token budget): per-head bounds,
    per-head Top-K, the union and the attention over it (8 rows of up to
    512 entries: 2 pages per wave, 64 splits, the wide merge), against the
    oracle on two sampled kv-heads."""
    wl = synth.Workload("gqa_union_32k", 1, 32, 8, (32768,), 2048, "f16",
                        outliers=4, base_seed=74)
    C.say(f"[case] {wl.name}: Hq 32 / Hkv 8, ctx 32768, union of per-head Top-K")
    c = build(wl)
    kv, k, G = c["kv"], wl.k_pages, 4
    kmin, kmax = C.gpu_meta(c)
    st = qa.UnionDecodeStep(kv, k, SM)
    out = st(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    heads = [1, 6]
    qh = [g * G + r for g in heads for r in range(G)]
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    lens = c["seq_lens"].cpu().numpy().astype(np.int64)
    q = C.to64(c["q"][:, qh])
    kp, vp = C.to64(c["k_pool"][:, heads]), C.to64(c["v_pool"][:, heads])
    omin, omax = O.page_meta(kp, pt, lens, 16)
    s_ora = O.estimate_heads(q, omin, omax, pt, lens, 16, kv.max_pages_per_seq)
    C.assert_scores_close(st.scores.cpu().numpy().astype(np.float64)[:, qh], s_ora, lens)
    sel_heads = st.sel_heads.cpu().numpy().astype(np.int64)[:, qh]
    C.assert_sets_match(sel_heads, s_ora, lens, k)
    sel = st.sel.cpu().numpy().astype(np.int64)[:, heads]
    assert np.array_equal(sel, O.union_pages(sel_heads, G))
    kept = [int((sel[0, i] >= 0).sum()) for i in range(len(heads))]
    C.say(f"  union keeps {kept} pages of {G * k} slots")
    ref = O.sparse_attention(q, kp, vp, pt, lens, sel, SM, 16)
    worst = C.assert_attention_close(out.cpu().numpy().astype(np.float64)[:, qh], ref)
    C.say(f"  union attention max err {worst:.2e}")


def test_page32_layer_128k():
    """32-token pages at 128K context with a 2048-token budget (64 pages of
    4096 per head), 32 heads, fp16."""
    wl = synth.Workload("p32_128k", 1, 32, 32, (131072,), 2048, "f16",
                        page_size=32, outliers=4, planted=5, base_seed=72)
    C.say(f"[case] {wl.name}: 32 heads, ctx 131072, 32-token pages, k={wl.k_pages}")
    c = build(wl)
    step, meta = run_paths(c, wl.k_pages)
    worst = check_units(c, step, [(0, [4]), (0, [29])], wl.k_pages, 1,
                        check_meta=meta, S=32)
    C.say(f"  sampled attention max err {worst:.2e}")


@pytest.mark.parametrize("path", ["calls", "append_step"])
def test_gqa_multistep_three_layers(path):
    """Layers 0-1 dense, layer 2 sparse (GQA 32/8, group score = sum of the 4
    query heads' bounds), three appended decode steps at 32K (the first
    append opens a new page), against the oracle's layer step on two
    sampled kv-heads.  "calls": the append by quest_update_page_meta, then
    the step; "append_step": the benchmark's own path -- the append folded
    into the bounds launch (quest_append_estimate), then the Top-K +
    attention call, and on the dense layers into the attention launch
    (quest_append_decode_attn)."""
    wl = synth.gqa_multistep_workload(layers=3, steps=3)
    G = wl.group
    heads = [1, 6]
    qh = [g * G + r for g in heads for r in range(G)]
    k = wl.k_pages
    C.say(f"[case] {wl.name}: 3 layers x 3 steps, Hq 32 / Hkv 8, ctx 32768")
    layers = []
    for layer in range(wl.layers):
        c = synth.draw_layer(wl, layer, "cuda")
        kv = qa.paged_kv(1, 32, 8, wl.pool_pages(), wl.max_pages, wl.torch_dtype)
        kmin, kmax = qa.alloc_meta(kv)
        qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                                  c["page_table"], c["seq_lens"])
        o = dict(kp=C.to64(c["k_pool"][:, heads]), vp=C.to64(c["v_pool"][:, heads]),
                 pt=c["page_table"].cpu().numpy().astype(np.int64))
        o["kmin"], o["kmax"] = O.page_meta(o["kp"], o["pt"],
                                           c["seq_lens"].cpu().numpy(), 16)
        layers.append(dict(c=c, kv=kv, kmin=kmin, kmax=kmax, o=o,
                           step=qa.SparseDecodeStep(kv, k, SM),
                           dense=qa.DenseDecode(kv, SM)))
    L = wl.seq_lens[0]
    for step in range(wl.steps):
        L += 1
        lens = torch.tensor([L], dtype=torch.int32, device="cuda")
        for layer, st in enumerate(layers):
            c, kv = st["c"], st["kv"]
            q = synth.draw_query(wl, layer, "cuda", step=step)
            k_new, v_new = synth.draw_append_token(wl, layer, step, "cuda")
            if path == "calls":
                qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], st["kmin"],
                                          st["kmax"], c["page_table"], lens,
                                          k_new=k_new, v_new=v_new)
            if layer < wl.dense_layers and path == "calls":
                out = st["dense"](q, c["k_pool"], c["v_pool"], c["page_table"], lens)
            elif layer < wl.dense_layers:
                out = st["dense"].append_step(q, c["k_pool"], c["v_pool"], st["kmin"],
                                              st["kmax"], c["page_table"], lens,
                                              k_new, v_new)
            elif path == "calls":
                out = st["step"](q, c["k_pool"], c["v_pool"], st["kmin"],
                                  st["kmax"], c["page_table"], lens)
            else:
                out = st["step"].append_step(q, c["k_pool"], c["v_pool"], st["kmin"],
                                             st["kmax"], c["page_table"], lens,
                                             k_new, v_new)
            torch.cuda.synchronize()
            o = st["o"]
            s_o, sel_o, out_o = O.layer_step(
                layer, wl.dense_layers, C.to64(q[:, qh]), o["kp"], o["vp"],
                o["kmin"], o["kmax"], o["pt"], np.array([L]),
                C.to64(k_new[:, heads]), C.to64(v_new[:, heads]), k, SM, 16)
            got = out.cpu().numpy().astype(np.float64)[:, qh]
            if layer < wl.dense_layers:
                C.assert_attention_close(got, out_o)
            else:
                f = st["step"]
                s_gpu = f.scores.cpu().numpy().astype(np.float64)[:, heads]
                C.assert_scores_close(s_gpu, s_o, np.array([L]))
                sel = f.sel.cpu().numpy().astype(np.int64)[:, heads]
                C.assert_sets_match(sel, s_o, np.array([L]), k)
                ref = O.sparse_attention(C.to64(q[:, qh]), o["kp"], o["vp"],
                                         o["pt"], np.array([L]), sel, SM, 16)
                C.assert_attention_close(got, ref)
    # boxes after the appends equal the oracle's running boxes, bit for bit
    for st in layers:
        n = -(-L // 16)
        pages = torch.tensor(st["o"]["pt"][0, :n].tolist(), dtype=torch.long)
        for gpu, ora in ((st["kmin"], st["o"]["kmin"]), (st["kmax"], st["o"]["kmax"])):
            g16 = gpu.cpu()[pages][:, heads].view(torch.int16)
            o16 = torch.from_numpy(ora[pages.numpy()]).to(gpu.dtype).view(torch.int16)
            assert torch.equal(g16, o16)
