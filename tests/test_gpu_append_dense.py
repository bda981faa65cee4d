"""quest_append_decode_attn (the step's token appended inside the dense
attention launch) against quest_update_page_meta (append mode) followed by
quest_decode_attn, over 20 appended tokens that cross page and tile
boundaries: K and V pools and boxes bit for bit, the attention up to the
order of its split sums (the two attention instances' plans need not split
the rows alike: each takes its own occupancy), and the last step's attention against the
oracle's dense attention ("Guide to Quest": §1 boxes, the attention
equation).  Every attention instance the append mode launches (both
dtypes, groups of 1, 2, 4 and 8, 16- and 32-token pages) is covered.
Also: appends whose page-table entry names no pool page are skipped by
both."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
import synth
from oracle import quest_oracle as O

import gpu_cases as C
from test_gpu_append_estimate import appended

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
STEPS = 20
CASES = {
    # name: (B, Hq, Hkv, lens, dtype, page_size)
    "mha_f16": (3, 4, 4, (1, 37, 1000), "f16", 16),
    "gqa2_bf16": (2, 8, 4, (15, 700), "bf16", 16),
    "gqa4_bf16": (2, 16, 4, (513, 2000), "bf16", 16),
    "gqa8_f16": (1, 16, 2, (1500,), "f16", 16),
    "with_empty": (3, 2, 2, (0, 33, 16), "f16", 16),
    "p32_mha_f16": (2, 4, 4, (31, 900), "f16", 32),
    "p32_gqa4_f16": (2, 16, 4, (95, 2000), "f16", 32),
}


def make(name):
    B, Hq, Hkv, lens, dt, S = CASES[name]
    wl = C.workload(B, Hq, Hkv, lens, 128, dt, 0, True, 4, 0, name, page_size=S)
    wl = dataclasses.replace(wl, steps=STEPS)     # pool and table hold the appends
    C.say(f"[case] append_decode_attn {name} lens={lens} S={S}")
    return wl, C.draw(wl)


def two_ways(wl, c):
    """Every step by update_page_meta (append) + decode_attn on the draw's
    buffers and by append_decode_attn on copies; the pools and boxes must
    agree bit for bit, the outputs up to the order of their split sums.
    Returns the last step's inputs and fused output."""
    kv = c["kv"]
    kmin_a, kmax_a = C.gpu_meta(c)
    kmin_b, kmax_b = kmin_a.clone(), kmax_a.clone()
    kp_a, vp_a = c["k_pool"], c["v_pool"]
    kp_b, vp_b = kp_a.clone(), vp_a.clone()
    dense_a, dense_b = qa.DenseDecode(kv, SM), qa.DenseDecode(kv, SM)
    i16 = lambda t: t.view(torch.int16)
    for step in range(STEPS):
        lens, k_new, v_new = appended(wl, c, step)
        q = synth.draw_query(wl, 0, "cuda", step=step)
        qa.quest_update_page_meta(kv, kp_a, vp_a, kmin_a, kmax_a, c["page_table"],
                                  lens, k_new=k_new, v_new=v_new)
        out_a = dense_a(q, kp_a, vp_a, c["page_table"], lens)
        out_b = dense_b.append_step(q, kp_b, vp_b, kmin_b, kmax_b, c["page_table"], lens,
                                    k_new, v_new)
        torch.cuda.synchronize()
        C.assert_same_up_to_split_order(out_a, out_b)
        assert torch.equal(i16(kmin_a), i16(kmin_b)) and \
            torch.equal(i16(kmax_a), i16(kmax_b)), step
    assert torch.equal(i16(kp_a), i16(kp_b)) and torch.equal(i16(vp_a), i16(vp_b))
    return q, kp_b, vp_b, lens, out_b


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_decode_attn_equals_two_calls(name):
    wl, c = make(name)
    q, kp, vp, lens, out = two_ways(wl, c)
    # the last step's attention against the oracle
    lens_h = lens.cpu().numpy().astype(np.int64)
    ref = O.dense_attention(C.to64(q), C.to64(kp), C.to64(vp),
                            c["page_table"].cpu().numpy().astype(np.int64), lens_h, SM,
                            wl.page_size)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("S", [16, 32])
def test_every_append_instance(S, G, dt):
    """Each attention instance the append mode launches (dtype x group size
    x page size), over appends that cross a page boundary, equals the two
    calls."""
    Hkv = 2
    lens = (S * 3 - 2, 5 * S + 7)                 # the first fills its page at step 1
    wl = C.workload(2, G * Hkv, Hkv, lens, 128, dt, 5 + G, True, 4, 0,
                    f"inst_{dt}_g{G}_p{S}", page_size=S)
    wl = dataclasses.replace(wl, steps=STEPS)
    C.say(f"[case] append_decode_attn instance S={S} G={G} {dt} lens={lens}")
    c = C.draw(wl)
    q, kp, vp, lens_t, out = two_ways(wl, c)
    ref = O.dense_attention(C.to64(q), C.to64(kp), C.to64(vp),
                            c["page_table"].cpu().numpy().astype(np.int64),
                            lens_t.cpu().numpy().astype(np.int64), SM, S)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("entry", ["negative", "past_pool"])
def test_append_into_an_absent_page(entry):
    """A request whose appended tokens land in pages whose table entries
    name no pool page appends nothing and attends over its other pages, in
    both compositions; the other requests append as usual."""
    wl, c = make("mha_f16")
    kv = c["kv"]
    r, S = 2, wl.page_size
    v = -1 if entry == "negative" else kv.num_pool_pages
    c["page_table"][r, wl.seq_lens[r] // S:] = v
    kp0 = c["k_pool"].clone()
    two_ways(wl, c)
    # request r wrote nowhere: the pools changed only in the slots the other
    # requests appended to
    changed = (c["k_pool"].view(torch.int16) != kp0.view(torch.int16)).any(dim=-1)
    pt = c["page_table"].cpu().numpy()
    others = {int(pt[b, (L + t) // S]) for b, L in enumerate(wl.seq_lens)
              if b != r and L > 0 for t in range(STEPS)}
    assert set(torch.nonzero(changed.flatten(1).any(dim=1)).flatten().tolist()) <= others
