"""The fused one-launch step (quest_sparse_decode_step) against the three
separate calls and the oracle: same scores and selection bit for bit, the
same attention within float32 rounding, and a workspace whose counters are
back at zero after every call."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C
from test_gpu_parity import CASES, make

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skip(reason="quest_sparse_decode_step is switched off: its "
                     "kernel did not complete on gfx950 (first runs timed out "
                     "in the first call); the cause is not yet found"),
]

SM = 1.0 / math.sqrt(128)


def run_both(c, k):
    kmin, kmax = C.gpu_meta(c)
    sep = qa.SparseDecodeStep(c["kv"], k, SM)
    fused = qa.FusedDecodeStep(c["kv"], k, SM)
    args = (c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
            c["seq_lens"])
    sep(*args)
    fused(*args)
    torch.cuda.synchronize()
    return sep, fused, kmin, kmax


@pytest.mark.parametrize("name", sorted(CASES))
def test_fused_equals_separate_and_oracle(name):
    wl, c = make(name)
    sep, fused, _, _ = run_both(c, wl.k_pages)
    assert torch.equal(fused.scores.view(torch.int32), sep.scores.view(torch.int32))
    assert torch.equal(fused.sel, sep.sel)
    err = (fused.out - sep.out).abs().max().item()
    assert err <= 1e-5, err
    assert fused.control_words().tolist() == [0, 0, 0]
    o = C.oracle_inputs(c)
    out_ora = O.sparse_attention(o["q"], o["k_pool"], o["v_pool"],
                                 o["page_table"], o["seq_lens"],
                                 fused.sel.cpu().numpy().astype(np.int64), SM, 16)
    C.assert_attention_close(fused.out.cpu().numpy().astype(np.float64), out_ora)


@pytest.mark.parametrize("k", [1, 3, 64, 10000])
def test_fused_budget_extremes(k):
    wl, c = make("gqa4_f16")
    sep, fused, _, _ = run_both(c, k)
    assert torch.equal(fused.sel, sep.sel)
    assert (fused.out - sep.out).abs().max().item() <= 1e-5
    assert fused.control_words().tolist() == [0, 0, 0]


def test_fused_repeated_calls_reuse_workspace():
    """Twenty calls on changing inputs through one workspace: every call
    matches the separate path, and the counters return to zero."""
    wl, c = make("mha_ragged_f16")
    kv = c["kv"]
    kmin, kmax = C.gpu_meta(c)
    sep = qa.SparseDecodeStep(kv, wl.k_pages, SM)
    fused = qa.FusedDecodeStep(kv, wl.k_pages, SM)
    g = torch.Generator(device="cuda").manual_seed(11)
    for i in range(20):
        q = torch.randn(c["q"].shape, generator=g, device="cuda").to(c["q"].dtype)
        args = (q, c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
                c["seq_lens"])
        sep(*args)
        fused(*args)
        torch.cuda.synchronize()
        assert torch.equal(fused.sel, sep.sel), i
        assert (fused.out - sep.out).abs().max().item() <= 1e-5, i
        assert fused.control_words().tolist() == [0, 0, 0], i
