"""The seeded generators: determinism, per-unit regeneration and the
structure the workloads ask for (outlier channels, planted pages, ragged
lengths, permuted pool)."""
import math

import numpy as np
import torch

import synth
from oracle import quest_oracle as O


def test_same_seed_same_bytes():
    wl = synth.tiny_workload()
    a = synth.draw_layer(wl, 0, "cpu")
    b = synth.draw_layer(wl, 0, "cpu")
    for k in a:
        assert torch.equal(a[k].view(torch.uint8) if a[k].is_floating_point()
                           else a[k], b[k].view(torch.uint8)
                           if b[k].is_floating_point() else b[k]), k


def test_unit_regenerates_alone():
    wl = synth.longchat_layer_workload(ctx=1024, budget=256)
    full = synth.draw_layer(wl, 0, "cpu", heads=[0, 1, 2])
    one = synth.draw_layer(wl, 0, "cpu", heads=[2])
    assert torch.equal(full["k_pool"][:, 2].view(torch.int16),
                       one["k_pool"][:, 2].view(torch.int16))


def test_tail_slots_are_nan_and_valid_finite():
    wl = synth.Workload("t", 2, 2, 2, (37, 16), 64, "bf16")
    c = synth.draw_layer(wl, 0, "cpu")
    for b, L in enumerate((37, 16)):
        n = -(-L // 16)
        for j in range(n):
            p = int(c["page_table"][b, j])
            v = min(16, L - 16 * j)
            assert torch.isfinite(c["k_pool"][p, :, :v].float()).all()
            assert torch.isnan(c["k_pool"][p, :, v:].float()).all()
            assert torch.isnan(c["v_pool"][p, :, v:].float()).all()


def test_outlier_channels_scaled():
    wl = synth.longchat_layer_workload(ctx=4096, budget=256)
    c = synth.draw_layer(wl, 0, "cpu", heads=[3])
    ch = synth.outlier_channels(wl, 0, 3)
    assert ch.numel() == 4
    k = c["k_pool"][:256, 3].float().reshape(-1, 128)
    plant = synth.planted_pages(wl, 0, 0, 3, 256)
    keep = torch.ones(256, dtype=torch.bool)
    keep[plant] = False
    k = c["k_pool"][:256, 3][keep].float().reshape(-1, 128)
    std = k.std(dim=0)
    others = torch.ones(128, dtype=torch.bool)
    others[ch] = False
    assert torch.all(std[ch] > 6.0) and torch.all(std[others] < 1.2)


def test_planted_pages_aligned_and_selected():
    """Planted keys sit at cosine ~0.9 to the head's query, and the oracle's
    Top-K keeps every planted page (a sanity check of the generator)."""
    wl = synth.longchat_layer_workload(ctx=32768, budget=2048)
    heads = [0, 17]
    c = synth.draw_layer(wl, 0, "cpu", heads=heads)
    q = c["q"].double().numpy()
    kp = c["k_pool"].double().numpy()
    pt = c["page_table"].numpy()
    lens = c["seq_lens"].numpy()
    kmin, kmax = O.page_meta(kp, pt, lens, 16)
    for g in heads:
        plant = synth.planted_pages(wl, 0, 0, g, 2048).numpy()
        assert len(plant) == 5
        qh = q[0, g] / np.linalg.norm(q[0, g])
        rows = kp[plant, g].reshape(-1, 128)
        cos = rows @ qh / np.linalg.norm(rows, axis=1)
        assert np.all(np.abs(cos - 0.9) < 0.01)
        pages = pt[0, :2048]
        s = np.maximum(q[0, g] * kmin[pages, g], q[0, g] * kmax[pages, g]).sum(1)
        sel = O.topk_pages(s, 2048, 128)
        assert set(plant) <= set(sel.tolist())


def test_ragged_and_permuted_pool():
    wl = synth.ragged_batch_workload()
    assert len(wl.seq_lens) == 32
    assert all(8192 <= L <= 32768 for L in wl.seq_lens)
    assert len(set(wl.seq_lens)) > 20
    pt = synth.page_table_for(wl)
    used = []
    for b, L in enumerate(wl.seq_lens):
        used += pt[b, :-(-L // 16)].tolist()
    assert sorted(used) == list(range(wl.pool_pages()))
    assert used != sorted(used)
    assert synth.ragged_batch_workload().seq_lens == wl.seq_lens


def test_append_tokens_follow_outliers():
    wl = synth.gqa_multistep_workload(layers=2, steps=4, ctx=64)
    k, v = synth.draw_append_token(wl, 1, 0, "cpu")
    assert k.shape == (1, 8, 128) and v.shape == (1, 8, 128)
    assert wl.max_pages == math.ceil((64 + 4) / 16)
    k2, _ = synth.draw_append_token(wl, 1, 0, "cpu")
    assert torch.equal(k.view(torch.int16), k2.view(torch.int16))
