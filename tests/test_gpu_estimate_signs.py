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
