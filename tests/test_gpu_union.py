"""The GQA union rule ("Guide to Quest", Best Practices 2) on the GPU:
per-query-head bounds against the oracle's estimate_heads, the union
kernel bit for bit against the oracle's union_pages, whole union steps
(per-head Top-K, union, attention over the union) against the oracle, with
the union built by its own launch or inside the attention launch, and the
latter (quest_union_sparse_decode_attn) bit for bit against the two calls."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C
from test_gpu_parity import make

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
GQA_CASES = ["gqa2_bf16", "gqa4_f16", "gqa8_f16", "mha_ragged_f16",
             "with_empty_request", "planted_f16"]


@pytest.mark.parametrize("name", GQA_CASES)
def test_estimate_heads_matches_oracle(name):
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s = torch.full((kv.batch, kv.num_q_heads, kv.max_pages_per_seq), 7.0,
                   device="cuda")
    qa.quest_estimate_heads(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], s)
    sg = torch.empty(kv.batch, kv.num_kv_heads, kv.max_pages_per_seq, device="cuda")
    qa.quest_estimate(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], sg)
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    s_ora = O.estimate_heads(o["q"], omin, omax, o["page_table"], o["seq_lens"],
                             16, kv.max_pages_per_seq)
    got = s.cpu().numpy().astype(np.float64)
    C.assert_scores_close(got, s_ora, o["seq_lens"])
    # the heads' rows add up to the group row (both float32 sums)
    G = kv.num_q_heads // kv.num_kv_heads
    grp = sg.cpu().numpy().astype(np.float64)
    for b, L in enumerate(o["seq_lens"]):
        n = -(-int(L) // 16)
        tot = got[b, :, :n].reshape(kv.num_kv_heads, G, n).sum(axis=1)
        assert np.all(np.abs(tot - grp[b, :, :n]) <=
                      2e-4 * np.abs(got[b, :, :n]).reshape(kv.num_kv_heads, G, n).sum(axis=1))


@pytest.mark.parametrize("G,k,mp", [(1, 8, 64), (2, 16, 300), (4, 128, 2048),
                                    (8, 40, 1000), (4, 512, 32768)])
def test_union_kernel_bitexact(G, k, mp):
    """Per-head lists with repeats across heads, -1 padding, short lists and
    out-of-range entries (which are ignored)."""
    B, Hkv = 3, 2
    Hq = G * Hkv
    rng = np.random.default_rng(G * 1000 + k)
    sel = np.full((B, Hq, k), -1, dtype=np.int32)
    for b in range(B):
        pool = rng.choice(mp, size=min(mp, 3 * k), replace=False)
        for h in range(Hq):
            m = int(rng.integers(0, k + 1))
            sel[b, h, :m] = np.sort(rng.choice(pool, size=min(m, len(pool)), replace=False))[:m]
    sel[0, 0, 0] = mp + 5            # out of range: ignored
    sel[1, -1, -1] = -3              # negative: ignored
    C.say(f"[case] union G={G} k={k} mp={mp}")
    kv = qa.paged_kv(B, Hq, Hkv, 1, mp, torch.float16)
    out = torch.full((B, Hkv, G * k), -7, dtype=torch.int32, device="cuda")
    qa.quest_union_pages(kv, torch.from_numpy(sel).cuda(), k, out)
    torch.cuda.synchronize()
    clean = np.where((sel >= 0) & (sel < mp), sel, -1)
    assert np.array_equal(out.cpu().numpy(), O.union_pages(clean, G))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("ns,nl", [(0, 0), (1, 2)])
@pytest.mark.parametrize("name", GQA_CASES)
def test_union_step_matches_oracle(name, ns, nl, fused):
    wl, c = make(name)
    kv = c["kv"]
    k = wl.k_pages
    G = kv.num_q_heads // kv.num_kv_heads
    kmin, kmax = C.gpu_meta(c)
    st = qa.UnionDecodeStep(kv, k, SM, n_sink=ns, n_local=nl, fused=fused)
    assert st.fused == fused
    if ns + nl > k:                      # a budget below the forced pages is refused
        with pytest.raises(qa.QuestError, match="n_sink"):
            st(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
               c["seq_lens"])
        return
    st.sel.fill_(-777)
    out = st(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
             c["seq_lens"])
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    s_ora = O.estimate_heads(o["q"], omin, omax, o["page_table"], o["seq_lens"],
                             16, kv.max_pages_per_seq)
    C.assert_scores_close(st.scores.cpu().numpy().astype(np.float64), s_ora,
                          o["seq_lens"])
    sel_heads = st.sel_heads.cpu().numpy().astype(np.int64)
    C.assert_sets_match(sel_heads, s_ora, o["seq_lens"], k, n_sink=ns, n_local=nl)
    sel = st.sel.cpu().numpy().astype(np.int64)
    assert np.array_equal(sel, O.union_pages(sel_heads, G))
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"], sel, SM, 16)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), out_ora)


def _random_head_lists(rng, B, Hq, k, lens, S, mp):
    """Per-head lists as a per-head Top-K leaves them (distinct, ascending,
    -1 padded, some short), drawn from a shared set of each request's pages
    so that heads repeat pages, plus entries past the request's end and
    entries outside [0, max_pages) that the union ignores."""
    sel = np.full((B, Hq, k), -1, dtype=np.int32)
    for b in range(B):
        n = max(1, -(-int(lens[b]) // S))
        pool = rng.choice(min(mp, n + 3), size=min(min(mp, n + 3), 3 * k), replace=False)
        for h in range(Hq):
            m = int(rng.integers(0, k + 1))
            pick = np.sort(rng.choice(pool, size=min(m, len(pool)), replace=False))
            sel[b, h, :len(pick)] = pick
    sel[0, 0, -1] = mp + 5
    sel[-1, -1, -1] = -3
    return sel


def _two_ways(kv, c, sel_heads, k):
    G = kv.num_q_heads // kv.num_kv_heads
    sh = torch.from_numpy(sel_heads).cuda()
    shape_u = (kv.batch, kv.num_kv_heads, G * k)
    shape_o = (kv.batch, kv.num_q_heads, kv.head_dim)
    u1 = torch.full(shape_u, -7, dtype=torch.int32, device="cuda")
    u2 = torch.full(shape_u, -9, dtype=torch.int32, device="cuda")
    o1 = torch.full(shape_o, 5.0, device="cuda")
    o2 = torch.full(shape_o, 6.0, device="cuda")
    ws1, ws2 = qa.alloc_workspace(kv, G * k), qa.alloc_workspace(kv, G * k)
    qa.quest_union_pages(kv, sh, k, u1)
    qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                                c["seq_lens"], u1, G * k, SM, o1, ws1)
    qa.quest_union_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                      c["page_table"], c["seq_lens"], sh, k, SM, u2, o2,
                                      ws2)
    torch.cuda.synchronize()
    assert torch.equal(u1, u2)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))
    return u2, o2


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("S", [16, 32])
def test_fused_union_attention_equals_two_calls(S, G, dt):
    lens = (700, 33, 1500, 0)
    wl = C.workload(4, 2 * G, 2, lens, 10 * S, dt, 30 + G, True, 4, 0,
                    f"union_fused_{dt}_g{G}_p{S}", page_size=S)
    C.say(f"[case] fused union S={S} G={G} {dt} lens={lens} k={wl.k_pages}")
    c = C.draw(wl)
    kv = c["kv"]
    rng = np.random.default_rng(S * 100 + G)
    sel = _random_head_lists(rng, kv.batch, kv.num_q_heads, wl.k_pages, lens, S,
                             kv.max_pages_per_seq)
    u, out = _two_ways(kv, c, sel, wl.k_pages)
    clean = np.where((sel >= 0) & (sel < kv.max_pages_per_seq), sel, -1)
    assert np.array_equal(u.cpu().numpy(), O.union_pages(clean, G))


@pytest.mark.parametrize("name,B,Hkv,G,k,lens,S", [
    # more rows than resident workgroups
    ("many_rows", 600, 4, 4, 16, None, 16),
    # 8 rows of 600 entries: 75 splits of 8 would leave a partial second
    # round, so the plan cuts them to one round and workgroups walk 2 chunks
    ("cut_ranges", 1, 8, 4, 150, (32768,), 16),
    # the longest list the attention workgroups build: G * k = 4096
    ("longest_list", 1, 1, 8, 512, (32768,), 16),
])
def test_fused_union_attention_shapes(name, B, Hkv, G, k, lens, S):
    rng = np.random.default_rng(B + k)
    if lens is None:
        lens = tuple(int(x) for x in rng.integers(1, 400, size=B))
    wl = C.workload(B, G * Hkv, Hkv, lens, k * S, "f16", 50, True, 0, 0, name,
                    page_size=S)
    C.say(f"[case] fused union {name} B={B} Hkv={Hkv} G={G} k={k}")
    c = C.draw(wl)
    kv = c["kv"]
    sel = _random_head_lists(rng, B, G * Hkv, k, lens, S, kv.max_pages_per_seq)
    _two_ways(kv, c, sel, k)
