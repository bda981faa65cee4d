"""GPU parity against the CPU oracle at sizes the oracle finishes in
seconds: several tiles, ragged tails, permuted pools, both dtypes, every
supported GQA group size, and the edge cases (empty and one-token requests,
k >= n, ties, signed zeros, NaN in unused slots)."""
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

CASES = {
    # name: (B, Hq, Hkv, lens, budget, dtype, permute, outliers, planted)
    "tiny_ref": (1, 1, 1, (1024,), 128, "f16", False, 0, 0),
    "mha_ragged_f16": (3, 4, 4, (1, 37, 1000), 160, "f16", True, 4, 0),
    "mha_ragged_bf16": (3, 4, 4, (16, 530, 777), 112, "bf16", True, 0, 0),
    "gqa2_bf16": (2, 8, 4, (300, 65), 64, "bf16", True, 0, 0),
    "gqa4_f16": (2, 16, 4, (513, 2000), 240, "f16", False, 4, 0),
    "gqa8_f16": (1, 16, 2, (1500,), 320, "f16", True, 0, 0),
    "planted_f16": (2, 8, 8, (4096, 3000), 256, "f16", False, 4, 5),
    "with_empty_request": (3, 2, 2, (0, 33, 16), 32, "f16", True, 0, 0),
    # rows of 2048..4096 pages (the 16-scores-per-thread Top-K variant)
    "gqa4_2500_pages": (1, 8, 2, (39990,), 512, "f16", True, 4, 0),
}


def make(name, seed=0):
    B, Hq, Hkv, lens, budget, dt, perm, outl, plant = CASES[name]
    wl = C.workload(B, Hq, Hkv, lens, budget, dt, seed, perm, outl, plant, name)
    C.say(f"[case] {name} seed={seed} B={B} Hq={Hq} Hkv={Hkv} lens={lens} "
          f"k={wl.k_pages} {dt}")
    return wl, C.draw(wl)


@pytest.mark.parametrize("name", sorted(CASES))
def test_meta_rebuild_bitexact(name):
    wl, c = make(name)
    kmin, kmax = C.gpu_meta(c)
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    pages = C.used_pages(o["page_table"], o["seq_lens"])
    C.assert_meta_bitexact(kmin, kmax, omin, omax, pages)


def test_meta_signed_zeros_and_extremes():
    for dt in (torch.float16, torch.bfloat16):
        C.say(f"[case] signed zeros {dt}")
        kv = qa.paged_kv(1, 1, 1, 2, 2, dt)
        k_pool = torch.full((2, 1, 16, 128), float("nan"), dtype=dt)
        vals = torch.tensor([-0.0, 0.0, -1e-7, 1e-7, -60000.0, 60000.0,
                             float("inf"), float("-inf")], dtype=dt)
        g = torch.Generator().manual_seed(5)
        for t in range(16):
            k_pool[0, 0, t] = vals[torch.randint(0, 8, (128,), generator=g)]
        k_pool[1, 0, :3] = vals[torch.randint(0, 2, (3, 128), generator=g)]
        lens = torch.tensor([19], dtype=torch.int32)
        pt = torch.tensor([[0, 1]], dtype=torch.int32)
        c = dict(kv=kv, k_pool=k_pool.cuda(), v_pool=k_pool.cuda(),
                 page_table=pt.cuda(), seq_lens=lens.cuda())
        kmin, kmax = C.gpu_meta(c)
        kp = k_pool.to(torch.float64).numpy()
        omin, omax = O.page_meta(kp, pt.numpy(), lens.numpy(), 16)
        C.assert_meta_bitexact(kmin, kmax, omin, omax, [0, 1])


@pytest.mark.parametrize("name", ["mha_ragged_f16", "gqa4_f16",
                                  "with_empty_request", "mha_ragged_bf16"])
def test_meta_append_and_partial_rebuild(name):
    """Appending the last tokens one at a time, and a rebuild that starts
    mid-sequence, both give the full rebuild's boxes bit for bit."""
    wl, c = make(name)
    full_lens = c["seq_lens"].clone()
    steps = 21
    start = torch.clamp(full_lens - steps, min=0)
    kv = c["kv"]
    ref_min, ref_max = C.gpu_meta(c)
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    pages = C.used_pages(o["page_table"], o["seq_lens"])
    C.assert_meta_bitexact(ref_min, ref_max, omin, omax, pages)

    # the tokens to append, read from the full pool, then removed from it
    pt = c["page_table"].long()
    B, H = kv.batch, kv.num_kv_heads
    kp = c["k_pool"].clone()
    vp = c["v_pool"].clone()
    news = []
    for s in range(steps):
        pos = start + s
        k_new = torch.zeros(B, H, 128, dtype=kp.dtype, device="cuda")
        v_new = torch.zeros_like(k_new)
        active = pos < full_lens
        for b in range(B):
            if active[b]:
                p = pt[b, pos[b] // 16]
                k_new[b] = kp[p, :, pos[b] % 16]
                v_new[b] = vp[p, :, pos[b] % 16]
        news.append((k_new, v_new, active))
    for b in range(B):
        for x in range(int(start[b]), int(full_lens[b])):
            kp[pt[b, x // 16], :, x % 16] = float("nan")
            vp[pt[b, x // 16], :, x % 16] = float("nan")

    # partial rebuild: boxes of [0, start), then fold [start, full) in place
    kmin, kmax = qa.alloc_meta(kv)
    kmin.fill_(float("nan"))
    kmax.fill_(float("nan"))
    qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                              c["page_table"], start.cuda())
    # first rebuild saw the full pool but only `start` tokens: fold the rest
    qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                              c["page_table"], full_lens, first_token=start.cuda())
    C.assert_meta_bitexact(kmin, kmax, omin, omax, pages)

    # append path
    amin, amax = qa.alloc_meta(kv)
    amin.fill_(float("nan"))
    amax.fill_(float("nan"))
    qa.quest_update_page_meta(kv, kp, vp, amin, amax, c["page_table"], start.cuda())
    lens = start.clone()
    for s, (k_new, v_new, active) in enumerate(news):
        lens = lens + active.to(torch.int32)
        # requests that are already complete pass L = 0 -> skipped
        L = torch.where(active, lens, torch.zeros_like(lens)).to(torch.int32)
        qa.quest_update_page_meta(kv, kp, vp, amin, amax, c["page_table"],
                                  L.cuda(), k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    C.assert_meta_bitexact(amin, amax, omin, omax, pages)
    for b in range(B):
        for x in range(int(full_lens[b])):
            p = pt[b, x // 16]
            assert torch.equal(kp[p, :, x % 16].view(torch.int16),
                               c["k_pool"][p, :, x % 16].view(torch.int16))
            assert torch.equal(vp[p, :, x % 16].view(torch.int16),
                               c["v_pool"][p, :, x % 16].view(torch.int16))


@pytest.mark.parametrize("name", sorted(CASES))
def test_estimate_matches_oracle(name):
    wl, c = make(name)
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    # feed the oracle's boxes (exact in the storage dtype) to the kernel
    dt = wl.torch_dtype
    kmin = torch.from_numpy(np.nan_to_num(omin, nan=0.0)).to(dt).cuda()
    kmax = torch.from_numpy(np.nan_to_num(omax, nan=0.0)).to(dt).cuda()
    kv = c["kv"]
    scores = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq),
                        12345.0, device="cuda")
    qa.quest_estimate(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"],
                      scores)
    torch.cuda.synchronize()
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                       kv.max_pages_per_seq)
    C.assert_scores_close(scores.cpu().numpy().astype(np.float64), s_ora,
                          o["seq_lens"])


def _topk_case(rows, n_list, mp, k, seed):
    """fp32 scores [B, 1, mp] with NaN beyond each row's n (must be ignored)."""
    g = np.random.default_rng(seed)
    s = np.full((rows, 1, mp), np.nan, dtype=np.float32)
    kinds = ["normal", "ties", "equal", "zeros", "inf", "sorted_up", "sorted_dn",
             "denormal", "extreme"]
    for r in range(rows):
        n = n_list[r]
        kind = kinds[r % len(kinds)]
        if kind == "normal":
            v = g.standard_normal(n).astype(np.float32) * 100
        elif kind == "ties":
            v = g.integers(-4, 5, n).astype(np.float32)
        elif kind == "equal":
            v = np.full(n, 3.5, dtype=np.float32)
        elif kind == "zeros":
            v = np.where(g.random(n) < 0.5, -0.0, 0.0).astype(np.float32)
            v[g.random(n) < 0.1] = 1e-30
        elif kind == "inf":
            v = g.standard_normal(n).astype(np.float32)
            v[g.random(n) < 0.3] = -np.inf
            v[g.random(n) < 0.05] = np.inf
        elif kind == "sorted_up":
            v = np.arange(n, dtype=np.float32)
        elif kind == "denormal":  # signed subnormals, signed zeros, ties among them
            tiny = np.float32(1.4e-45)
            v = (g.integers(-40, 41, n) * tiny).astype(np.float32)
            v[g.random(n) < 0.2] = -0.0
        elif kind == "extreme":  # the ends of the float32 range and its neighbours
            pool = np.array([np.finfo(np.float32).max, -np.finfo(np.float32).max,
                             np.nextafter(np.finfo(np.float32).max, np.float32(0)),
                             np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny,
                             1.0, -1.0, np.inf, -np.inf], dtype=np.float32)
            v = pool[g.integers(0, len(pool), n)]
        else:
            v = -np.arange(n, dtype=np.float32)
        s[r, 0, :n] = v
    return s


@pytest.mark.parametrize("mp,k", [(64, 8), (1024, 100), (1027, 100), (2048, 128),
                                  (4100, 256), (8192, 512), (16384, 1000),
                                  (32768, 4096)])
def test_topk_kernel_bitexact(mp, k):
    rows = 14
    g = np.random.default_rng(mp + k)
    n_list = [mp, k, k + 1, max(1, k - 1), 0, 1] + \
        [int(x) for x in g.integers(1, mp + 1, rows - 6)]
    C.say(f"[case] topk mp={mp} k={k} n={n_list}")
    s = _topk_case(rows, n_list, mp, k, seed=mp)
    lens = torch.tensor([n * 16 for n in n_list], dtype=torch.int32)
    kv = qa.paged_kv(rows, 1, 1, 1, mp, torch.float16)
    sel = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    qa.quest_topk_pages(kv, torch.from_numpy(s).cuda(), lens.cuda(), k, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for r in range(rows):
        ref = O.topk_pages(s[r, 0].astype(np.float64), n_list[r], k)
        assert np.array_equal(got[r, 0], ref), f"row {r} n={n_list[r]}"


@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_sparse_step_matches_oracle(name, select):
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s_gpu, sel_gpu, out_gpu = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM,
                                             select=select)
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                       kv.max_pages_per_seq)
    C.assert_scores_close(s_gpu, s_ora, o["seq_lens"])
    C.assert_sets_match(sel_gpu, s_ora, o["seq_lens"], wl.k_pages)
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"], sel_gpu, SM, 16)
    err = C.assert_attention_close(out_gpu, out_ora)
    C.say(f"  attention max err {err:.2e}")
    if wl.planted:
        for b in range(kv.batch):
            for g in range(kv.num_kv_heads):
                plant = set(int(x) for x in synth.planted_pages(
                    wl, 0, b, g, int(o["seq_lens"][b]) // 16))
                assert plant <= set(sel_gpu[b, g].tolist())


@pytest.mark.parametrize("name", sorted(CASES))
def test_dense_matches_oracle(name):
    wl, c = make(name)
    dense = qa.DenseDecode(c["kv"], SM)
    out = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    ref = O.dense_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                            o["seq_lens"], SM, 16)
    err = C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)
    C.say(f"  dense max err {err:.2e}")


@pytest.mark.parametrize("name", ["tiny_ref", "gqa4_f16", "mha_ragged_bf16"])
def test_full_budget_sparse_equals_dense(name):
    """k >= n_b keeps every page: the sparse call is full attention."""
    wl, c = make(name)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    k = kv.max_pages_per_seq + 3
    _, sel, out = C.run_gpu_step(c, k, kmin, kmax, SM)
    dense = qa.DenseDecode(kv, SM)
    d = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    for b, L in enumerate(c["seq_lens"].tolist()):
        n = -(-L // 16)
        assert np.array_equal(sel[b, :, :n], np.tile(np.arange(n), (kv.num_kv_heads, 1)))
    assert np.max(np.abs(out - d.cpu().numpy())) <= 1e-5


def test_step_is_deterministic():
    """100 repeats of the step give the same scores, selection and output
    bit for bit (no atomics, fixed split and merge order)."""
    wl, c = make("gqa4_f16")
    kmin, kmax = C.gpu_meta(c)
    first = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM)
    for _ in range(100):
        again = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM)
        for a, b in zip(first, again):
            assert np.array_equal(a, b, equal_nan=True)


def test_sparse_selection_order_irrelevant():
    """The attention call accepts any order of the listed pages and -1
    holes anywhere."""
    wl, c = make("mha_ragged_f16")
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    _, sel, out = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM)
    rng = np.random.default_rng(3)
    shuffled = sel.copy()
    for b in range(sel.shape[0]):
        for g in range(sel.shape[1]):
            shuffled[b, g] = shuffled[b, g][rng.permutation(sel.shape[2])]
    o2 = torch.empty_like(torch.from_numpy(out).float()).cuda()
    ws = qa.alloc_workspace(kv, wl.k_pages)
    qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                c["page_table"], c["seq_lens"],
                                torch.from_numpy(shuffled).int().cuda(),
                                wl.k_pages, SM, o2, ws)
    torch.cuda.synchronize()
    assert np.max(np.abs(o2.cpu().numpy() - out)) <= 1e-5


def test_workspace_reuse_is_stateless():
    """Reusing one workspace across calls (and filling it with garbage in
    between) changes nothing: the attention calls keep no state in it."""
    wl, c = make("gqa4_f16")
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    step = qa.SparseDecodeStep(kv, wl.k_pages, SM)
    dense = qa.DenseDecode(kv, SM)
    args = (c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
            c["seq_lens"])
    first = step(*args).clone()
    d_first = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                    c["seq_lens"]).clone()
    for i in range(5):
        step.workspace.fill_(0xA5 + i)
        dense.workspace.fill_(0x5A + i)
        step(*args)
        dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
        torch.cuda.synchronize()
        assert torch.equal(step.out, first)
        assert torch.equal(dense.out, d_first)


@pytest.mark.parametrize("k_extra", [None, 1, 2, 5, 10000])
@pytest.mark.parametrize("name", sorted(CASES))
def test_topk_attn_equals_separate_calls(name, k_extra):
    """quest_topk_sparse_decode_attn == quest_topk_pages then
    quest_sparse_decode_attn: the same selection bit for bit (and every slot
    of sel_pages written, which starts out full of a sentinel), the same
    output up to the float32 rounding of a different split and merge order."""
    wl, c = make(name)
    k = wl.k_pages if k_extra is None else k_extra
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    a = qa.SparseDecodeStep(kv, k, SM, select="attention")
    b = qa.SparseDecodeStep(kv, k, SM, select="separate")
    if a.select != "attention":
        pytest.skip("beyond the one-launch Top-K size limit")
    a.sel.fill_(-777)
    args = (c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
            c["seq_lens"])
    a(*args)
    b(*args)
    torch.cuda.synchronize()
    assert int((a.sel == -777).sum()) == 0
    assert torch.equal(a.sel, b.sel)
    C.assert_same_up_to_split_order(a.out, b.out)


@pytest.mark.parametrize("k_extra", [None, 1, 5])
@pytest.mark.parametrize("name", ["tiny_ref", "mha_ragged_f16", "gqa4_f16",
                                  "gqa8_f16", "with_empty_request"])
def test_topk_attn_splits_then_merge_equals_one_call(name, k_extra):
    """quest_topk_sparse_decode_attn_splits followed by
    quest_merge_attn_splits launch the same two kernels as
    quest_topk_sparse_decode_attn_ex: sel_pages and out bit for bit (also
    when the plan has a single split, where the first call writes out and
    the merge does nothing), with forced pages too."""
    wl, c = make(name)
    k = wl.k_pages if k_extra is None else k_extra
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    for n_sink, n_local in ((0, 0), (1, min(2, k - 1))):
        a = qa.SparseDecodeStep(kv, k, SM, select="attention", n_sink=n_sink,
                                n_local=n_local)
        a(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"], c["seq_lens"])
        sel = torch.full_like(a.sel, -777)
        out = torch.full_like(a.out, float("nan"))
        ws = qa.alloc_workspace(kv, k)
        qa.quest_topk_sparse_decode_attn_splits(
            kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"],
            a.scores, k, n_sink, n_local, SM, sel, out, ws)
        qa.quest_merge_attn_splits(kv, k, ws, out)
        torch.cuda.synchronize()
        assert torch.equal(sel, a.sel)
        assert torch.equal(out.view(torch.int32), a.out.view(torch.int32))


@pytest.mark.parametrize("select", ["attention", "separate"])
def test_graph_replay_matches_eager(select):
    """The step captured in a HIP graph: every replay, with eager work and
    synchronisations in between and new queries copied in, equals an eager
    step on the same inputs."""
    wl, c = make("mha_ragged_f16")
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    step = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    ref = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    q = c["q"].clone()
    args = lambda qq: (qq, c["k_pool"], c["v_pool"], kmin, kmax,
                       c["page_table"], c["seq_lens"])
    step(*args(q))                      # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(*args(q))
    gen = torch.Generator(device="cuda").manual_seed(3)
    for i in range(5):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref(*args(q))                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(step.sel, ref.sel), i
        assert torch.equal(step.out.view(torch.int32), ref.out.view(torch.int32)), i
        assert torch.equal(step.scores.view(torch.int32), ref.scores.view(torch.int32)), i


@pytest.mark.parametrize("mp,rows", [(2056, 12), (2056, 300), (4104, 12), (1027, 300),
                                     (2048, 300), (2560, 12), (2561, 12), (2560, 300)])
def test_topk_segment_boundaries(mp, rows):
    """Rows whose length crosses the 4-page segments of the selection's key
    layout (1024, 2048 and 4096 pages and just past them) and the one-key
    tail after 2048 pages (rows of up to 2560), with few rows (the 8-wave
    launch, keys in segments of 4) and many (the 4-wave one, keys in runs):
    bit-exact against the oracle, every score kind."""
    k = 128
    g = np.random.default_rng(mp * 7 + rows)
    edges = [n for n in (1023, 1024, 1025, 1028, 2047, 2048, 2049, 2052, 2056, 2559,
                         2560, 2561, 4095, 4096, 4097, 4100, 4104) if n <= mp]
    n_list = (edges * (rows // len(edges) + 1))[:rows]
    n_list[-1] = int(g.integers(1, mp + 1))
    C.say(f"[case] topk segments mp={mp} rows={rows}")
    s = _topk_case(rows, n_list, mp, k, seed=mp + rows)
    lens = torch.tensor([n * 16 for n in n_list], dtype=torch.int32)
    kv = qa.paged_kv(rows, 1, 1, 1, mp, torch.float16)
    sel = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    qa.quest_topk_pages(kv, torch.from_numpy(s).cuda(), lens.cuda(), k, sel)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for r in range(rows):
        ref = O.topk_pages(s[r, 0].astype(np.float64), n_list[r], k)
        assert np.array_equal(got[r, 0], ref), f"row {r} n={n_list[r]}"


@pytest.mark.parametrize("mp", [2056, 2560, 2561, 4104])
def test_topk_attn_selection_segment_boundaries(mp):
    """The selection inside the attention launch (quest_topk_sparse_decode_attn,
    keys in segments of 4, with a one-key tail for rows of up to 2560 pages)
    at lengths around the segment boundaries: its sel_pages output bit-exact
    against the oracle."""
    rows, k = 12, 128
    edges = [n for n in (2047, 2048, 2049, 2052, 2056, 2559, 2560, 2561, 4096, 4097,
                         4104, 1, 129) if n <= mp]
    n_list = (edges * 2)[:rows]
    C.say(f"[case] topk_attn segments mp={mp} n={n_list}")
    s = _topk_case(rows, n_list, mp, k, seed=mp + 11)
    s = np.nan_to_num(s, nan=0.0)  # the fused call reads its own rows only up to n
    kv = qa.paged_kv(rows, 1, 1, mp, mp, torch.float16)
    lens = torch.tensor([n * 16 for n in n_list], dtype=torch.int32, device="cuda")
    pt = torch.arange(mp, dtype=torch.int32, device="cuda").repeat(rows, 1).contiguous()
    q = torch.randn(rows, 1, 128, device="cuda").half()
    kp = torch.randn(mp, 1, 16, 128, device="cuda").half()
    vp = torch.randn(mp, 1, 16, 128, device="cuda").half()
    out = torch.empty(rows, 1, 128, device="cuda")
    sel = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    ws = qa.alloc_workspace(kv, k)
    qa.quest_topk_sparse_decode_attn(kv, q, kp, vp, pt, lens, torch.from_numpy(s).cuda(),
                                     k, SM, sel, out, ws)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    for r in range(rows):
        ref = O.topk_pages(s[r, 0].astype(np.float64), n_list[r], k)
        assert np.array_equal(got[r, 0], ref), f"row {r} n={n_list[r]}"
