"""Seeded random geometries through the whole sparse step, against the
oracle: group size, dtype, page size, ragged lengths on and around page
edges, empty and one-token requests, budgets below and above the page
count, forced sink / local pages, the softmax scale, and page tables wider
than the longest request whose unused entries hold garbage (negative ids,
ids past the pool, ids of other requests' pages).  Every fifth case has a
row of more than 2048 pages (the wider Top-K variants).

For each case: metadata bit for bit; bounds within 1e-4 relative; the
Top-K set equal to the oracle's (forced pages included) up to swaps within
1e-4 relative; sparse and dense attention within 2e-3 absolute.  The
selection inside the attention launch and the separate Top-K launch must
give the same scores and lists and the same output up to the float32
order of the split merge."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

N_CASES = 25


def _lengths(rng, B, S, long_row):
    lens = []
    for b in range(B):
        if long_row and b == 0:
            n = int(rng.integers(2049, (6000 if S == 16 else 4500) + 1))
            lens.append(n * S - int(rng.integers(0, S)))
            continue
        kind = rng.choice(["one", "edge", "random", "empty"], p=[0.15, 0.35, 0.4, 0.1])
        if kind == "empty" and B > 1:
            lens.append(0)
        elif kind == "one":
            lens.append(1)
        elif kind == "edge":
            lens.append(max(1, int(rng.integers(1, 120)) * S + int(rng.integers(-1, 2))))
        else:
            lens.append(int(rng.integers(1, 3001)))
    return tuple(lens)


def geometry(i):
    rng = np.random.default_rng(7100 + i)
    long_row = i % 5 == 4
    S = int(rng.choice([16, 32]))
    G = int(rng.choice([1, 2, 4, 8]))
    if long_row:
        B, Hkv = 1, 1
    else:
        B, Hkv = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3]))
    lens = _lengths(rng, B, S, long_row)
    n_max = max(1, max(-(-L // S) for L in lens))
    k = int(rng.integers(1, n_max + 4))
    n_sink = n_local = 0
    if rng.random() < 0.35:
        n_sink = int(rng.integers(0, 3))
        n_local = int(rng.integers(0, 4))
        while n_sink + n_local > k:
            if n_local > 0:
                n_local -= 1
            else:
                n_sink -= 1
    return dict(seed=7100 + i, S=S, G=G, B=B, Hkv=Hkv, lens=lens, k=k,
                n_sink=n_sink, n_local=n_local,
                dtype=str(rng.choice(["f16", "bf16"])),
                permute=bool(rng.random() < 0.5),
                outliers=int(rng.choice([0, 4])),
                extra=int(rng.integers(0, 50)),
                sm=float(rng.choice([0.5, 1.0, 2.0])) / math.sqrt(128),
                rng=rng)


def widen_table(c, geo, pool_pages):
    """A [B][n_max + extra] table: the drawn entries below each request's
    page count, garbage everywhere else."""
    rng = geo["rng"]
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    B, mp0 = pt.shape
    S = geo["S"]
    mp = mp0 + geo["extra"]
    out = rng.integers(-5, pool_pages + 5, size=(B, mp))
    wild = rng.random((B, mp)) < 0.1
    out[wild] = rng.choice([-2**31, 2**31 - 1, -1, pool_pages], size=int(wild.sum()))
    for b, L in enumerate(geo["lens"]):
        n = -(-L // S)
        out[b, :n] = pt[b, :n]
    return torch.from_numpy(out.astype(np.int32)).cuda(), mp


def setup(i, what):
    geo = geometry(i)
    S, G, B, Hkv = geo["S"], geo["G"], geo["B"], geo["Hkv"]
    wl = C.workload(B, Hkv * G, Hkv, geo["lens"], geo["k"] * S, geo["dtype"],
                    geo["seed"], geo["permute"], geo["outliers"], 0,
                    f"random_{i}", page_size=S)
    C.say(f"[case] random geometry {i} ({what}): S={S} G={G} B={B} Hkv={Hkv} "
          f"lens={geo['lens']} k={geo['k']} sink={geo['n_sink']} "
          f"local={geo['n_local']} {geo['dtype']} extra={geo['extra']}")
    c = C.draw(wl)
    c["page_table"], mp = widen_table(c, geo, wl.pool_pages())
    c["kv"] = qa.paged_kv(B, Hkv * G, Hkv, wl.pool_pages(), mp, wl.torch_dtype,
                          page_size=S)
    return geo, wl, c, mp


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_geometry_step(i):
    geo, wl, c, mp = setup(i, "step")
    S, kv = geo["S"], c["kv"]
    kmin, kmax = C.gpu_meta(c)

    res = {}
    for select in ("attention", "separate"):
        step = qa.SparseDecodeStep(kv, geo["k"], geo["sm"], select=select,
                                   n_sink=geo["n_sink"], n_local=geo["n_local"])
        out = step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
                   c["seq_lens"])
        res[select] = (step.scores.clone(), step.sel.clone(), out.clone())
    dense = qa.DenseDecode(kv, geo["sm"])
    d = dense(c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()

    # the two placements of the Top-K agree exactly on scores and lists
    sa, la, oa = res["attention"]
    ss, ls, os_ = res["separate"]
    assert torch.equal(sa.view(torch.int32), ss.view(torch.int32))
    assert torch.equal(la, ls)
    C.assert_same_up_to_split_order(oa, os_)

    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], S)
    C.assert_meta_bitexact(kmin, kmax, omin, omax,
                           C.used_pages(o["page_table"], o["seq_lens"], S))
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], S, mp)
    s_gpu = sa.cpu().numpy().astype(np.float64)
    C.assert_scores_close(s_gpu, s_ora, o["seq_lens"], S)
    sel = la.cpu().numpy().astype(np.int64)
    swaps = C.assert_sets_match(sel, s_ora, o["seq_lens"], geo["k"], S,
                                geo["n_sink"], geo["n_local"])
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                                 o["seq_lens"], sel, geo["sm"], S)
    err = C.assert_attention_close(oa.cpu().numpy().astype(np.float64), out_ora)
    ref = O.dense_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                            o["seq_lens"], geo["sm"], S)
    derr = C.assert_attention_close(d.cpu().numpy().astype(np.float64), ref)
    C.say(f"  swaps {swaps}, sparse err {err:.2e}, dense err {derr:.2e}")


@pytest.mark.parametrize("i", range(0, N_CASES, 3))
def test_random_geometry_append(i):
    """Boxes built up to L - 1, then the step that appends token L - 1 (the
    pool's own row, so the pools keep their contents) together with the
    bounds: boxes, bounds, lists and output bit for bit those of the plain
    step on the full rebuild."""
    geo, wl, c, mp = setup(i, "append")
    S, kv = geo["S"], c["kv"]
    full_min, full_max = C.gpu_meta(c)
    lens = c["seq_lens"]
    prev = torch.clamp(lens - 1, min=0)
    kmin, kmax = qa.alloc_meta(kv)
    kmin.fill_(float("nan"))
    kmax.fill_(float("nan"))
    qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                              c["page_table"], prev)
    B, Hkv = kv.batch, kv.num_kv_heads
    k_new = torch.zeros(B, Hkv, 128, dtype=c["k_pool"].dtype, device="cuda")
    v_new = torch.zeros_like(k_new)
    pt = c["page_table"].long()
    for b, L in enumerate(lens.tolist()):
        if L > 0:
            p = pt[b, (L - 1) // S]
            k_new[b] = c["k_pool"][p, :, (L - 1) % S]
            v_new[b] = c["v_pool"][p, :, (L - 1) % S]
    kp0, vp0 = c["k_pool"].clone(), c["v_pool"].clone()
    args = dict(n_sink=geo["n_sink"], n_local=geo["n_local"])
    step = qa.SparseDecodeStep(kv, geo["k"], geo["sm"], **args)
    out = step.append_step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax,
                           c["page_table"], lens, k_new, v_new)
    ref = qa.SparseDecodeStep(kv, geo["k"], geo["sm"], **args)
    ref_out = ref(c["q"], kp0, vp0, full_min, full_max, c["page_table"], lens)
    torch.cuda.synchronize()
    assert torch.equal(c["k_pool"].view(torch.int16), kp0.view(torch.int16))
    assert torch.equal(c["v_pool"].view(torch.int16), vp0.view(torch.int16))
    pages = C.used_pages(c["page_table"].cpu().numpy(), lens.tolist(), S)
    idx = torch.tensor(pages, dtype=torch.long, device="cuda")
    for a, r in ((kmin, full_min), (kmax, full_max)):
        assert torch.equal(a[idx].view(torch.int16), r[idx].view(torch.int16))
    assert torch.equal(step.scores.view(torch.int32), ref.scores.view(torch.int32))
    assert torch.equal(step.sel, ref.sel)
    assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32))
