"""quest_append_estimate == quest_update_page_meta (append) + quest_estimate,
bit for bit (scores, boxes, K and V pools), over 20 appended tokens that
cross page boundaries, also when the appended tokens' page-table entries
name no pool page (both skip those appends), in every bounds instance the
append mode launches; and SparseDecodeStep.append_step equals the two-call
composition."""
import dataclasses
import math

import pytest
import torch

import query_aware_kv_amd as qa
import synth

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
STEPS = 20
CASES = {
    # name: (B, Hq, Hkv, lens, budget, dtype, page_size)
    "mha_f16": (3, 4, 4, (1, 37, 1000), 160, "f16", 16),
    "gqa4_bf16": (2, 16, 4, (513, 2000), 240, "bf16", 16),
    "gqa8_f16": (1, 16, 2, (1500,), 320, "f16", 16),
    "with_empty": (3, 2, 2, (0, 33, 16), 32, "f16", 16),
    "p32_gqa4_f16": (2, 16, 4, (95, 2000), 480, "f16", 32),
}


def make(name):
    B, Hq, Hkv, lens, budget, dt, S = CASES[name]
    wl = C.workload(B, Hq, Hkv, lens, budget, dt, 0, True, 4, 0, name, page_size=S)
    wl = dataclasses.replace(wl, steps=STEPS)     # pool and table hold the appends
    C.say(f"[case] append_estimate {name} lens={lens} S={S}")
    return wl, C.draw(wl)


def appended(wl, c, step):
    """The step's lengths (L = 0 requests stay empty) and its new K/V rows."""
    base = torch.tensor(wl.seq_lens, dtype=torch.int32)
    lens = torch.where(base > 0, base + step + 1, base).to(torch.int32).cuda()
    k_new, v_new = synth.draw_append_token(wl, 0, step, "cuda")
    return lens, k_new, v_new


def two_ways(wl, c):
    """Every step by update_page_meta (append) + estimate on the draw's
    buffers and by append_estimate on copies: scores, boxes and pools must
    agree bit for bit."""
    kv = c["kv"]
    kmin_a, kmax_a = C.gpu_meta(c)
    kmin_b, kmax_b = kmin_a.clone(), kmax_a.clone()
    kp_a, vp_a = c["k_pool"], c["v_pool"]
    kp_b, vp_b = kp_a.clone(), vp_a.clone()
    shape = (kv.batch, kv.num_kv_heads, kv.max_pages_per_seq)
    s_a = torch.empty(shape, device="cuda")
    s_b = torch.empty(shape, device="cuda")
    i16 = lambda t: t.view(torch.int16)
    for step in range(STEPS):
        lens, k_new, v_new = appended(wl, c, step)
        q = synth.draw_query(wl, 0, "cuda", step=step)
        qa.quest_update_page_meta(kv, kp_a, vp_a, kmin_a, kmax_a, c["page_table"],
                                  lens, k_new=k_new, v_new=v_new)
        qa.quest_estimate(kv, q, kmin_a, kmax_a, c["page_table"], lens, s_a)
        qa.quest_append_estimate(kv, kp_b, vp_b, kmin_b, kmax_b, c["page_table"],
                                 lens, k_new, v_new, q, s_b)
        torch.cuda.synchronize()
        assert torch.equal(s_a.view(torch.int32), s_b.view(torch.int32)), step
        assert torch.equal(i16(kmin_a), i16(kmin_b)) and \
            torch.equal(i16(kmax_a), i16(kmax_b)), step
    assert torch.equal(i16(kp_a), i16(kp_b)) and torch.equal(i16(vp_a), i16(vp_b))
    return s_b


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_estimate_equals_two_calls(name):
    wl, c = make(name)
    two_ways(wl, c)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("Hkv", [2, 4])          # 16-row and four-head mappings
@pytest.mark.parametrize("S", [16, 32])
def test_every_append_instance(S, Hkv, G, dt):
    """Each bounds instance the append mode launches (dtype x group size x
    work mapping, both page sizes), over appends that cross a page
    boundary, equals the two calls bit for bit."""
    lens = (S * 3 - 2, 5 * S + 7)                 # the first fills its page at step 1
    wl = C.workload(2, G * Hkv, Hkv, lens, 128, dt, 5 + G, True, 4, 0,
                    f"est_inst_{dt}_g{G}_h{Hkv}_p{S}", page_size=S)
    wl = dataclasses.replace(wl, steps=STEPS)
    C.say(f"[case] append_estimate instance S={S} Hkv={Hkv} G={G} {dt} lens={lens}")
    two_ways(wl, C.draw(wl))


@pytest.mark.parametrize("entry", ["negative", "past_pool"])
def test_append_into_an_absent_page(entry):
    """A request whose appended tokens land in pages whose table entries
    name no pool page appends nothing and scores those pages -inf, in both
    compositions; the other requests append as usual."""
    wl, c = make("mha_f16")
    kv = c["kv"]
    r, S = 2, wl.page_size
    v = -1 if entry == "negative" else kv.num_pool_pages
    first = wl.seq_lens[r] // S
    c["page_table"][r, first:] = v
    kp0 = c["k_pool"].clone()
    scores = two_ways(wl, c)
    assert torch.isneginf(scores[r, :, first:]).all()
    changed = (c["k_pool"].view(torch.int16) != kp0.view(torch.int16)).flatten(1).any(dim=1)
    pt = c["page_table"].cpu().numpy()
    others = {int(pt[b, (L + t) // S]) for b, L in enumerate(wl.seq_lens)
              if b != r and L > 0 for t in range(STEPS)}
    assert set(torch.nonzero(changed).flatten().tolist()) <= others


@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("name", ["gqa4_bf16", "p32_gqa4_f16"])
def test_append_step_equals_composition(name, select):
    wl, c = make(name)
    kv = c["kv"]
    kmin_a, kmax_a = C.gpu_meta(c)
    kmin_b, kmax_b = kmin_a.clone(), kmax_a.clone()
    kp_b, vp_b = c["k_pool"].clone(), c["v_pool"].clone()
    a = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    b = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    for step in range(5):
        lens, k_new, v_new = appended(wl, c, step)
        q = synth.draw_query(wl, 0, "cuda", step=step)
        qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin_a, kmax_a,
                                  c["page_table"], lens, k_new=k_new, v_new=v_new)
        a(q, c["k_pool"], c["v_pool"], kmin_a, kmax_a, c["page_table"], lens)
        b.append_step(q, kp_b, vp_b, kmin_b, kmax_b, c["page_table"], lens, k_new, v_new)
        torch.cuda.synchronize()
        assert torch.equal(a.sel, b.sel)
        assert torch.equal(a.out.view(torch.int32), b.out.view(torch.int32))
