"""The matrix-core attention of a GQA group (G >= 2 query heads per kv-head)
against two independent references: the oracle, and the VALU path of the
same library run one query head at a time (G = 1 views of the same pools).
Ragged lengths leave partial last pages whose unused slots hold NaN; a
scaled query makes the softmax peak sharply, so the online rescaling across
tiles, waves and splits carries the result."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)


def draw(G, dtype, S, lens, seed, q_gain=1.0, budget_pages=4):
    Hkv = 2
    wl = C.workload(len(lens), Hkv * G, Hkv, lens, budget_pages * S, dtype, seed, True, 4,
                    0, f"mfma_g{G}", page_size=S)
    C.say(f"[case] mfma G={G} {dtype} S={S} lens={lens} seed={seed} q_gain={q_gain}")
    c = C.draw(wl)
    if q_gain != 1.0:
        c["q"] = (c["q"].float() * q_gain).to(c["q"].dtype)
    return wl, c


def per_head_dense(c, G):
    """Dense attention of every query head of the group through G = 1
    descriptors over the same pools (the VALU path)."""
    kv = c["kv"]
    B, Hq, Hkv = kv.batch, kv.num_q_heads, kv.num_kv_heads
    kv1 = qa.paged_kv(B, Hkv, Hkv, kv.num_pool_pages, kv.max_pages_per_seq,
                      kv.torch_dtype, page_size=kv.page_size)
    out = torch.empty(B, Hq, 128, device="cuda")
    for h in range(G):
        q1 = c["q"].view(B, Hkv, G, 128)[:, :, h].contiguous()
        d = qa.DenseDecode(kv1, SM)
        o1 = d(q1, c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
        out.view(B, Hkv, G, 128)[:, :, h] = o1
    return out


@pytest.mark.parametrize("S", [16, 32])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [2, 4, 8])
def test_group_dense_matches_single_heads_and_oracle(G, dtype, S):
    wl, c = draw(G, dtype, S, (1, 17, 300, 1000), seed=G)
    kv = c["kv"]
    out = qa.DenseDecode(kv, SM)(c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                                 c["seq_lens"]).clone()
    ref1 = per_head_dense(c, G)
    torch.cuda.synchronize()
    err = float((out - ref1).abs().max())
    assert err <= 1e-5, f"MFMA group vs per-head VALU: {err:.3g}"
    o = C.oracle_inputs(c)
    ora = O.dense_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                            o["seq_lens"], SM, S)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ora)


@pytest.mark.parametrize("G", [2, 4, 8])
@pytest.mark.parametrize("select", ["attention", "separate"])
def test_group_sparse_sharp_softmax(G, select):
    """q scaled x30: a few tokens dominate each head's softmax, from pages
    spread over different splits."""
    wl, c = draw(G, "bf16", 16, (700, 2500), seed=100 + G, q_gain=30.0, budget_pages=64)
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    s_gpu, sel_gpu, out_gpu = C.run_gpu_step(c, wl.k_pages, kmin, kmax, SM, select=select)
    o = C.oracle_inputs(c)
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                                 o["seq_lens"], sel_gpu, SM, 16)
    C.assert_attention_close(out_gpu, out_ora)


def test_group_one_token_and_identical_keys():
    """A 1-token request attends to its one token (o = v_0); a page whose
    tokens share one key averages its values."""
    G = 4
    wl, c = draw(G, "f16", 16, (1, 16), seed=7)
    kv = c["kv"]
    # request 1: every key of its one page equal -> o = mean of V
    p1 = int(c["page_table"][1, 0])
    c["k_pool"][p1] = c["k_pool"][p1, :, :1].expand(-1, 16, -1)
    out = qa.DenseDecode(kv, SM)(c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                                 c["seq_lens"]).cpu().double()
    p0 = int(c["page_table"][0, 0])
    v = c["v_pool"].cpu().double()
    for g in range(kv.num_kv_heads):
        for h in range(G):
            assert torch.allclose(out[0, g * G + h], v[p0, g, 0], atol=1e-6)
            assert torch.allclose(out[1, g * G + h], v[p1, g].mean(0), atol=1e-5)
