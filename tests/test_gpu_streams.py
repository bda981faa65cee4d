"""The library keeps no state between calls: host threads that each drive
their own stream and buffers get, bit for bit, what the same calls give
when made one at a time on one stream."""
import math
import threading

import pytest
import torch

import query_aware_kv_amd as qa

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
REPS = 20
SHAPES = [
    # (B, Hq, Hkv, lens, budget, dtype, select)
    (2, 16, 4, (513, 2000), 240, "f16", "attention"),
    (3, 4, 4, (16, 530, 777), 112, "bf16", "separate"),
    (1, 8, 8, (4096,), 256, "f16", "attention"),
]


def _case(i):
    B, Hq, Hkv, lens, budget, dt, select = SHAPES[i]
    wl = C.workload(B, Hq, Hkv, lens, budget, dt, seed=300 + i, permute=True,
                    outliers=4, name=f"streams_{i}")
    c = C.draw(wl)
    kmin, kmax = C.gpu_meta(c)
    return wl, c, kmin, kmax, select


def _run(case, reps):
    wl, c, kmin, kmax, select = case
    step = qa.SparseDecodeStep(c["kv"], wl.k_pages, SM, select=select)
    res = []
    for _ in range(reps):
        out = step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
                   c["seq_lens"])
        res.append((out.clone(), step.sel.clone(), step.scores.clone()))
    return res


def test_threads_on_their_own_streams_match_serial_calls():
    C.say(f"[case] {len(SHAPES)} host threads x {REPS} steps, one stream each")
    cases = [_case(i) for i in range(len(SHAPES))]
    torch.cuda.synchronize()
    ref = [_run(cs, 1)[0] for cs in cases]
    torch.cuda.synchronize()

    results = [None] * len(cases)
    errors = []
    start = threading.Barrier(len(cases))

    def work(i):
        try:
            s = torch.cuda.Stream()  # default priority
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                start.wait()
                results[i] = _run(cases[i], REPS)
            s.synchronize()
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (out, sel, scores) in enumerate(ref):
        for r, (o2, s2, sc2) in enumerate(results[i]):
            assert torch.equal(o2.view(torch.int32), out.view(torch.int32)), (i, r)
            assert torch.equal(s2, sel), (i, r)
            assert torch.equal(sc2.view(torch.int32), scores.view(torch.int32)), (i, r)
