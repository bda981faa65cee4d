"""Decode steps that append a token, replayed from one captured HIP graph.

Before each replay the step's query, new K/V rows and lengths are copied
into the graph's input buffers, and eager work and synchronisations run
between replays.  Every replay's output, kept lists and bounds, and the
pools and boxes at the end, must equal eager steps on twin buffers bit for
bit.  Covers the sparse append step (quest_append_estimate, then the Top-K
and attention) and a dense layer of the multi-layer step, both as two calls
(the append in quest_update_page_meta, then quest_decode_attn) and as one
(quest_append_decode_attn).  The graph is warmed up
with the first step's inputs, which its first replay appends again:
appending the same token twice leaves the same pools and boxes."""
import dataclasses
import math

import pytest
import torch

import query_aware_kv_amd as qa
import synth

import gpu_cases as C

pytestmark = pytest.mark.gpu

SM = 1.0 / math.sqrt(128)
STEPS = 12


def _setup(S):
    wl = C.workload(2, 16, 4, (513, 1999), 240 if S == 16 else 480, "f16", seed=41,
                    permute=True, outliers=4, name=f"graph_append_p{S}", page_size=S)
    wl = dataclasses.replace(wl, steps=STEPS)  # pool and table hold the appends
    c = C.draw(wl)
    return wl, c


def _appended(wl, step):
    base = torch.tensor(wl.seq_lens, dtype=torch.int32)
    lens = torch.where(base > 0, base + step + 1, base).to(torch.int32).cuda()
    k_new, v_new = synth.draw_append_token(wl, 0, step, "cuda")
    q = synth.draw_query(wl, 0, "cuda", step=step)
    return lens, k_new, v_new, q


def _i16(t):
    return t.view(torch.int16)


def _i32(t):
    return t.view(torch.int32)


@pytest.mark.parametrize("select", ["attention", "separate"])
@pytest.mark.parametrize("S", [16, 32])
def test_sparse_append_steps_from_a_graph(S, select):
    wl, c = _setup(S)
    kv = c["kv"]
    C.say(f"[case] graph append sparse S={S} {select} lens={wl.seq_lens} steps={STEPS}")
    kmin_a, kmax_a = C.gpu_meta(c)
    kmin_b, kmax_b = kmin_a.clone(), kmax_a.clone()
    kp_a, vp_a = c["k_pool"], c["v_pool"]
    kp_b, vp_b = kp_a.clone(), vp_a.clone()
    pt = c["page_table"]
    a = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)
    b = qa.SparseDecodeStep(kv, wl.k_pages, SM, select=select)

    lens0, k0, v0, q0 = _appended(wl, 0)
    lens_g, knew_g, vnew_g, q_g = lens0.clone(), k0.clone(), v0.clone(), q0.clone()
    a.append_step(q_g, kp_a, vp_a, kmin_a, kmax_a, pt, lens_g, knew_g, vnew_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.append_step(q_g, kp_a, vp_a, kmin_a, kmax_a, pt, lens_g, knew_g, vnew_g)

    for step in range(STEPS):
        lens, k_new, v_new, q = _appended(wl, step)
        lens_g.copy_(lens)
        knew_g.copy_(k_new)
        vnew_g.copy_(v_new)
        q_g.copy_(q)
        g.replay()
        torch.cuda.synchronize()
        b.append_step(q, kp_b, vp_b, kmin_b, kmax_b, pt, lens, k_new, v_new)
        torch.cuda.synchronize()
        assert torch.equal(_i32(a.scores), _i32(b.scores)), step
        assert torch.equal(a.sel, b.sel), step
        assert torch.equal(_i32(a.out), _i32(b.out)), step
    assert torch.equal(_i16(kp_a), _i16(kp_b)) and torch.equal(_i16(vp_a), _i16(vp_b))
    assert torch.equal(_i16(kmin_a), _i16(kmin_b)) and torch.equal(_i16(kmax_a), _i16(kmax_b))


@pytest.mark.parametrize("path", ["calls", "fused"])
@pytest.mark.parametrize("S", [16, 32])
def test_dense_append_steps_from_a_graph(S, path):
    wl, c = _setup(S)
    kv = c["kv"]
    C.say(f"[case] graph append dense S={S} {path} lens={wl.seq_lens} steps={STEPS}")
    kmin_a, kmax_a = C.gpu_meta(c)
    kmin_b, kmax_b = kmin_a.clone(), kmax_a.clone()
    kp_a, vp_a = c["k_pool"], c["v_pool"]
    kp_b, vp_b = kp_a.clone(), vp_a.clone()
    pt = c["page_table"]
    a = qa.DenseDecode(kv, SM)
    b = qa.DenseDecode(kv, SM)

    def layer(d, q, kp, vp, kmin, kmax, lens, k_new, v_new):
        if path == "fused":
            return d.append_step(q, kp, vp, kmin, kmax, pt, lens, k_new, v_new)
        qa.quest_update_page_meta(kv, kp, vp, kmin, kmax, pt, lens,
                                  k_new=k_new, v_new=v_new)
        return d(q, kp, vp, pt, lens)

    lens0, k0, v0, q0 = _appended(wl, 0)
    lens_g, knew_g, vnew_g, q_g = lens0.clone(), k0.clone(), v0.clone(), q0.clone()
    layer(a, q_g, kp_a, vp_a, kmin_a, kmax_a, lens_g, knew_g, vnew_g)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_a = layer(a, q_g, kp_a, vp_a, kmin_a, kmax_a, lens_g, knew_g, vnew_g)

    for step in range(STEPS):
        lens, k_new, v_new, q = _appended(wl, step)
        lens_g.copy_(lens)
        knew_g.copy_(k_new)
        vnew_g.copy_(v_new)
        q_g.copy_(q)
        g.replay()
        torch.cuda.synchronize()
        out_b = layer(b, q, kp_b, vp_b, kmin_b, kmax_b, lens, k_new, v_new)
        torch.cuda.synchronize()
        assert torch.equal(_i32(out_a), _i32(out_b)), step
    assert torch.equal(_i16(kp_a), _i16(kp_b)) and torch.equal(_i16(vp_a), _i16(vp_b))
    assert torch.equal(_i16(kmin_a), _i16(kmin_b)) and torch.equal(_i16(kmax_a), _i16(kmax_b))
