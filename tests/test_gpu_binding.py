"""The Python binding checks every tensor's device, dtype, shape and
contiguity against the geometry before it calls the library, and raises
ValueError without launching anything (the output buffers keep their
contents)."""
import math

import pytest
import torch

import query_aware_kv_amd as qa

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def case():
    wl = C.workload(2, 8, 4, (300, 65), 64, "f16", seed=5, name="binding")
    c = C.draw(wl)
    kmin, kmax = C.gpu_meta(c)
    kv = c["kv"]
    scores = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), 7.0,
                        device="cuda")
    sel = torch.full((kv.batch, kv.num_kv_heads, wl.k_pages), -7, dtype=torch.int32,
                     device="cuda")
    out = torch.full((kv.batch, kv.num_q_heads, 128), 7.0, device="cuda")
    ws = qa.alloc_workspace(kv, wl.k_pages)
    torch.cuda.synchronize()
    return dict(wl=wl, c=c, kv=kv, kmin=kmin, kmax=kmax, scores=scores, sel=sel,
                out=out, ws=ws)


def _untouched(case):
    torch.cuda.synchronize()
    assert torch.all(case["scores"] == 7.0)
    assert torch.all(case["sel"] == -7)
    assert torch.all(case["out"] == 7.0)


def test_estimate_argument_checks(case):
    c, kv = case["c"], case["kv"]
    args = dict(q=c["q"], kmin=case["kmin"], kmax=case["kmax"],
                page_table=c["page_table"], seq_lens=c["seq_lens"],
                scores=case["scores"])
    bad = {
        "q": c["q"].float(),                                # dtype
        "kmin": case["kmin"][:-1],                          # shape
        "kmax": case["kmax"].transpose(0, 1),               # not contiguous
        "page_table": c["page_table"].long(),               # dtype
        "seq_lens": c["seq_lens"].cpu(),                    # device
        "scores": case["scores"][:, :, :-1],                # shape (and layout)
    }
    for name, t in bad.items():
        a = dict(args, **{name: t})
        with pytest.raises(ValueError, match=name):
            qa.quest_estimate(kv, a["q"], a["kmin"], a["kmax"], a["page_table"],
                              a["seq_lens"], a["scores"])
    _untouched(case)


def test_topk_and_attention_argument_checks(case):
    c, kv, k = case["c"], case["kv"], case["wl"].k_pages
    with pytest.raises(ValueError, match="sel_pages"):
        qa.quest_topk_pages(kv, case["scores"], c["seq_lens"], k, case["sel"][:, :, :-1])
    with pytest.raises(ValueError, match="scores"):
        qa.quest_topk_pages(kv, case["scores"].half(), c["seq_lens"], k, case["sel"])
    with pytest.raises(ValueError, match="out"):
        qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                    c["page_table"], c["seq_lens"], case["sel"], k,
                                    SM, case["out"].half(), case["ws"])
    with pytest.raises(ValueError, match="k_pool"):
        qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"].bfloat16(), c["v_pool"],
                                    c["page_table"], c["seq_lens"], case["sel"], k,
                                    SM, case["out"], case["ws"])
    with pytest.raises(ValueError, match="sel_pages"):
        qa.quest_topk_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                         c["page_table"], c["seq_lens"], case["scores"],
                                         k, SM, case["sel"].long(), case["out"], case["ws"])
    with pytest.raises(ValueError, match="v_pool"):
        qa.quest_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"][:1], c["page_table"],
                             c["seq_lens"], SM, case["out"], case["ws"])
    _untouched(case)
