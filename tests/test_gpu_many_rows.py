"""The largest grids the library accepts: 65520 (request, kv-head) rows
(4095 requests x 16 kv-heads, one to three pages each; the limit is 65535
rows), for query groups of 1 and 4, through the whole sparse step with the
Top-K in its own launch and inside the attention launch.  Sampled requests
are checked against the oracle (their pages copied into a compact pool);
every row is checked for a valid selection."""
import math

import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
B, HKV, K = 4095, 16, 2


_CACHES = {}


def _case(G):
    """One draw per group size, shared by both placements of the Top-K."""
    if G not in _CACHES:
        _CACHES.clear()
        rng = np.random.default_rng(77 + G)
        lens = tuple(int(x) for x in rng.integers(1, 49, size=B))
        wl = C.workload(B, HKV * G, HKV, lens, K * 16, "f16", seed=78 + G,
                        permute=True, name=f"max_rows_g{G}")
        C.say(f"  drawing {B} requests x {HKV} kv-heads (G={G})")
        c = C.draw(wl)
        kmin, kmax = C.gpu_meta(c)
        _CACHES[G] = (lens, c, kmin, kmax, rng)
    return _CACHES[G]


@pytest.mark.parametrize("select", ["separate", "attention"])
@pytest.mark.parametrize("G", [1, 4])
def test_max_rows_step(G, select):
    C.say(f"[case] {B} x {HKV} rows (G={G}, {select}), lengths 1..48, k={K}")
    lens, c, kmin, kmax, rng = _case(G)
    kv = c["kv"]
    step = qa.SparseDecodeStep(kv, K, SM, select=select)
    assert step.select == select
    step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    sel = step.sel.cpu().numpy().astype(np.int64)
    for b, L in enumerate(lens):
        n = -(-L // 16)
        for g in range(HKV):
            C.assert_valid_selection(sel[b, g], n, K)

    reqs = sorted(set([0, B - 1] + rng.choice(B, 10, replace=False).tolist()))
    C.say(f"  oracle on requests {reqs}")
    pt_all = c["page_table"].cpu().numpy().astype(np.int64)
    pages = [pt_all[b, :-(-lens[b] // 16)] for b in reqs]
    idx = torch.from_numpy(np.concatenate(pages)).cuda()
    kp, vp = C.to64(c["k_pool"][idx]), C.to64(c["v_pool"][idx])
    pt = np.zeros((len(reqs), kv.max_pages_per_seq), dtype=np.int64)
    off = 0
    for i, p in enumerate(pages):
        pt[i, :len(p)] = np.arange(off, off + len(p))
        off += len(p)
    sub_lens = np.array([lens[b] for b in reqs], dtype=np.int64)
    q = C.to64(c["q"][reqs])
    omin, omax = O.page_meta(kp, pt, sub_lens, 16)
    s_ora = O.estimate(q, omin, omax, pt, sub_lens, 16, kv.max_pages_per_seq)
    s_gpu = step.scores.cpu().numpy().astype(np.float64)[reqs]
    C.assert_scores_close(s_gpu, s_ora, sub_lens)
    C.assert_sets_match(sel[reqs], s_ora, sub_lens, K)
    out_ora = O.sparse_attention(q, kp, vp, pt, sub_lens, sel[reqs], SM, 16)
    err = C.assert_attention_close(step.out.cpu().numpy().astype(np.float64)[reqs],
                                   out_ora)
    C.say(f"  sampled requests {reqs}: attention max err {err:.2e}")
