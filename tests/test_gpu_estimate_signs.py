"""The estimate's per-channel bound max(q_i kmin_i, q_i kmax_i) is evaluated
as q_i times the corner of the box that the sign of q_i picks.  These cases
exercise that choice against the oracle's max form: query entries that are
+0, -0, negative or positive; box channels whose corners are -0 and +0; and
degenerate channels with kmin = kmax.  Group sums and per-head rows, fp16
and bf16, a partial last page and a one-token request."""
import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu


def _case(G, dtype):
    Hkv = 2
    wl = C.workload(2, Hkv * G, Hkv, (333, 1), 64, dtype, seed=50 + G, outliers=4,
                    name=f"signs_g{G}")
    C.say(f"[case] estimate signs G={G} {dtype} lens=(333, 1)")
    c = C.draw(wl)
    rng = np.random.default_rng(900 + G)
    q = C.to64(c["q"])
    r = rng.random(q.shape)
    q[r < 0.33] = 0.0
    q[(r >= 0.33) & (r < 0.43)] = -0.0
    c["q"] = torch.from_numpy(q).to(wl.torch_dtype).cuda()
    o = C.oracle_inputs(c)
    kmin, kmax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    kmin, kmax = np.nan_to_num(kmin, nan=0.0), np.nan_to_num(kmax, nan=0.0)
    used = C.used_pages(o["page_table"], o["seq_lens"])
    for p in used[::3]:  # corners -0 and +0
        ch = rng.choice(128, 16, replace=False)
        kmin[p][:, ch] = -0.0
        kmax[p][:, ch] = 0.0
    for p in used[1::3]:  # degenerate channels
        ch = rng.choice(128, 16, replace=False)
        kmax[p][:, ch] = kmin[p][:, ch]
    assert np.all(kmin <= kmax)
    dt = wl.torch_dtype
    return wl, c, o, kmin, kmax, torch.from_numpy(kmin).to(dt).cuda(), \
        torch.from_numpy(kmax).to(dt).cuda()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 4])
def test_estimate_sign_corners(G, dtype):
    wl, c, o, omin, omax, kmin, kmax = _case(G, dtype)
    kv = c["kv"]
    s = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), 12345.0,
                   device="cuda")
    qa.quest_estimate(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], s)
    sh = torch.full((kv.batch, kv.num_q_heads, kv.max_pages_per_seq), 12345.0,
                    device="cuda")
    qa.quest_estimate_heads(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], sh)
    torch.cuda.synchronize()
    ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                     kv.max_pages_per_seq)
    C.assert_scores_close(s.cpu().numpy().astype(np.float64), ora, o["seq_lens"])
    ora_h = O.estimate_heads(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                             kv.max_pages_per_seq)
    C.assert_scores_close(sh.cpu().numpy().astype(np.float64), ora_h, o["seq_lens"])


def test_estimate_all_zero_query_scores_zero():
    """q = 0 (either sign) makes every product zero: every score is 0."""
    wl, c, o, omin, omax, kmin, kmax = _case(4, "f16")
    kv = c["kv"]
    q = torch.zeros_like(c["q"])
    q.view(torch.int16)[..., ::2] = -0x8000  # -0 in every other channel
    s = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), 12345.0,
                   device="cuda")
    qa.quest_estimate(kv, q, kmin, kmax, c["page_table"], c["seq_lens"], s)
    torch.cuda.synchronize()
    for b, L in enumerate(o["seq_lens"]):
        n = -(-int(L) // 16)
        assert torch.all(s[b, :, :n] == 0.0)
        assert torch.all(torch.isneginf(s[b, :, n:]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_estimate_and_attention_with_subnormal_keys(dtype):
    """Keys scaled into the 16-bit subnormal range (fp16: below 2^-14): the
    boxes, the bounds and the attention must use their exact values (no
    flush to zero of 16-bit inputs)."""
    G = 4
    wl = C.workload(2, 4 * G, 4, (333, 64), 64, dtype, seed=60, name="subnormal")
    C.say(f"[case] subnormal keys {dtype}")
    c = C.draw(wl)
    # keys subnormal in their dtype; q scaled so that every product is a
    # normal float32 number
    k_scale, q_scale = (2.0 ** -20, 8.0) if dtype == "f16" else (2.0 ** -130, 2.0 ** 100)
    c["k_pool"] = (c["k_pool"].float() * k_scale).to(wl.torch_dtype)
    c["q"] = (c["q"].float() * q_scale).to(wl.torch_dtype)
    o = C.oracle_inputs(c)
    used = C.used_pages(o["page_table"], o["seq_lens"])
    kp = o["k_pool"][used]
    tiny = np.finfo(np.float16).tiny if dtype == "f16" else 2.0 ** -126
    frac = np.mean((np.abs(kp) < tiny) & (kp != 0))
    assert frac > 0.5, f"only {frac:.2f} of the keys are subnormal"
    kmin, kmax = C.gpu_meta(c)
    omin, omax = O.page_meta(o["k_pool"], o["page_table"], o["seq_lens"], 16)
    C.assert_meta_bitexact(kmin, kmax, omin, omax, used)
    kv = c["kv"]
    s = torch.empty((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), device="cuda")
    qa.quest_estimate(kv, c["q"], kmin, kmax, c["page_table"], c["seq_lens"], s)
    torch.cuda.synchronize()
    ora = O.estimate(o["q"], omin, omax, o["page_table"], o["seq_lens"], 16,
                     kv.max_pages_per_seq)
    C.assert_scores_close(s.cpu().numpy().astype(np.float64), ora, o["seq_lens"])
    # attention over every page: the logits are tiny, the output the mean of V
    step = qa.SparseDecodeStep(kv, kv.max_pages_per_seq, 1.0 / np.sqrt(128))
    out = step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
               c["seq_lens"])
    torch.cuda.synchronize()
    ref = O.dense_attention(o["q"], o["k_pool"], o["v_pool"], o["page_table"],
                            o["seq_lens"], 1.0 / np.sqrt(128), 16)
    C.assert_attention_close(out.cpu().numpy().astype(np.float64), ref)
