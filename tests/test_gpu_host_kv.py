"""K/V pools in pinned host memory ("Guide to Quest": the full cache stays
in host or device memory and only the critical pages are loaded): every
call that reads or writes the pools gives bit-identical results when the
pools live in host memory and the kernels read them over the host link."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa

import gpu_cases as C
from test_gpu_parity import make as make16
from test_gpu_page32 import make as make32

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


def host_pools(c):
    return qa.host_pool_like(c["k_pool"]), qa.host_pool_like(c["v_pool"])


@pytest.mark.parametrize("maker,name", [(make16, "mha_ragged_f16"),
                                        (make16, "gqa4_f16"),
                                        (make16, "with_empty_request"),
                                        (make32, "p32_gqa8_bf16")])
def test_host_pools_match_device_pools(maker, name):
    wl, c = maker(name)
    kv = c["kv"]
    hk, hv = host_pools(c)
    dmin, dmax = C.gpu_meta(c)
    hmin, hmax = qa.alloc_meta(kv)
    qa.quest_update_page_meta(kv, hk, hv, hmin, hmax, c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    o_pages = C.used_pages(c["page_table"].cpu().numpy(), c["seq_lens"].cpu().numpy(),
                           kv.page_size)
    idx = torch.tensor(o_pages, dtype=torch.long, device="cuda")
    assert torch.equal(hmin[idx].view(torch.int16), dmin[idx].view(torch.int16))
    assert torch.equal(hmax[idx].view(torch.int16), dmax[idx].view(torch.int16))
    for select in qa.SELECT_MODES:
        a = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
        b = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
        a(c["q"], c["k_pool"], c["v_pool"], dmin, dmax, c["page_table"], c["seq_lens"])
        b(c["q"], hk, hv, dmin, dmax, c["page_table"], c["seq_lens"])
        torch.cuda.synchronize()
        assert torch.equal(a.sel, b.sel)
        assert torch.equal(a.out.view(torch.int32), b.out.view(torch.int32))
    d1 = qa.DenseDecode(kv, SM)(c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                                c["seq_lens"]).clone()
    d2 = qa.DenseDecode(kv, SM)(c["q"], hk, hv, c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))


@pytest.mark.parametrize("how", ["update_page_meta", "append_estimate",
                                 "append_decode_attn"])
def test_append_into_host_pool(how):
    """Each append (the append kernel, and the appends inside the bounds and
    the dense attention launches) writes host pools as it writes device
    pools: the same boxes, slots and outputs, bit for bit."""
    wl, c = make16("gqa4_f16")
    kv = c["kv"]
    C.say(f"[case] append into host pools via {how}")
    hk, hv = host_pools(c)
    kmin, kmax = C.gpu_meta(c)
    # one more token for requests whose last page has room (others pass
    # L = 0, which the append skips)
    old = c["seq_lens"]
    lens = torch.where(old % 16 != 0, old + 1, torch.zeros_like(old)).to(torch.int32)
    assert int((lens > 0).sum()) > 0
    g = torch.Generator(device="cuda").manual_seed(9)
    k_new = torch.randn(kv.batch, kv.num_kv_heads, 128, generator=g,
                        device="cuda").to(c["k_pool"].dtype)
    v_new = torch.randn(kv.batch, kv.num_kv_heads, 128, generator=g,
                        device="cuda").to(c["k_pool"].dtype)
    pt = c["page_table"]
    dk, dv = c["k_pool"].clone(), c["v_pool"].clone()
    dmin, dmax = kmin.clone(), kmax.clone()

    def call(kp, vp, bmin, bmax):
        if how == "update_page_meta":
            qa.quest_update_page_meta(kv, kp, vp, bmin, bmax, pt, lens,
                                      k_new=k_new, v_new=v_new)
            return None
        if how == "append_estimate":
            scores = torch.empty(kv.batch, kv.num_kv_heads, kv.max_pages_per_seq,
                                 device="cuda")
            qa.quest_append_estimate(kv, kp, vp, bmin, bmax, pt, lens, k_new, v_new,
                                     c["q"], scores)
            return scores
        return qa.DenseDecode(kv, SM).append_step(c["q"], kp, vp, bmin, bmax, pt, lens,
                                                  k_new, v_new)

    r_dev = call(dk, dv, dmin, dmax)
    r_host = call(hk, hv, kmin, kmax)
    torch.cuda.synchronize()
    if r_dev is not None:
        assert torch.equal(r_dev.view(torch.int32), r_host.view(torch.int32))
    assert torch.equal(kmin.view(torch.int16), dmin.view(torch.int16))
    assert torch.equal(kmax.view(torch.int16), dmax.view(torch.int16))
    pt_h = pt.cpu().long()
    for b, L in enumerate(lens.cpu().tolist()):
        if L == 0:
            continue
        p, slot = pt_h[b, (L - 1) // 16], (L - 1) % 16
        assert torch.equal(hk.tensor[p, :, slot].view(torch.int16),
                           dk[p, :, slot].cpu().view(torch.int16))
        assert torch.equal(hv.tensor[p, :, slot].view(torch.int16),
                           dv[p, :, slot].cpu().view(torch.int16))
        assert torch.equal(hk.tensor[p, :, slot].view(torch.int16),
                           k_new[b].cpu().view(torch.int16))


@pytest.mark.parametrize("maker,name", [(make16, "gqa4_f16"), (make16, "mha_ragged_f16"),
                                        (make32, "p32_gqa8_bf16")])
def test_host_pool_step_against_oracle(maker, name):
    """The whole step with both pools in pinned host memory (boxes built
    from the host pools too), checked against the oracle directly rather
    than against the device-pool run: scores within 1e-4 relative, the
    Top-K set up to near-tie swaps, attention within 2e-3 on the GPU's own
    set."""
    from oracle import quest_oracle as O
    wl, c = maker(name)
    kv = c["kv"]
    S = kv.page_size
    hk, hv = host_pools(c)
    hmin, hmax = qa.alloc_meta(kv)
    qa.quest_update_page_meta(kv, hk, hv, hmin, hmax, c["page_table"], c["seq_lens"])
    step = qa.SparseDecodeStep(kv, wl.k_pages, SM)
    out = step(c["q"], hk, hv, hmin, hmax, c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    o = C.oracle_inputs(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], S)
    s_ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], S,
                       kv.max_pages_per_seq)
    C.assert_scores_close(step.scores.cpu().numpy().astype(np.float64), s_ora,
                          o["seq_lens"], S)
    sel = step.sel.cpu().numpy().astype(np.int64)
    C.assert_sets_match(sel, s_ora, o["seq_lens"], wl.k_pages, S)
    ref = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                             o["seq_lens"], sel, SM, S)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)
