"""quest_append_decode_attn (the step's token appended inside the dense
attention launch) against quest_update_page_meta (append mode) followed by
quest_decode_attn, over 20 appended tokens that cross page and tile
boundaries: K and V pools and boxes bit for bit, the attention up to the
order of its split sums (the append kernel holds more registers, so its plan
may split the rows differently), and the last step's attention against the
oracle's dense attention ("Guide to Quest": §1 boxes, the attention
equation)."""
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


@pytest.mark.parametrize("name", sorted(CASES))
def test_append_decode_attn_equals_two_calls(name):
    wl, c = make(name)
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
    # the last step's attention against the oracle
    lens_h = lens.cpu().numpy().astype(np.int64)
    ref = O.dense_attention(C.to64(q), C.to64(kp_b), C.to64(vp_b),
                            c["page_table"].cpu().numpy().astype(np.int64), lens_h, SM,
                            wl.page_size)
    C.assert_attention_close(out_b.cpu().numpy().astype(np.float64), ref)
