"""The union benchmark's attention-recall metric (bench.attention_recall)
on a hand-sized case, against a direct NumPy evaluation of its definition:
the full-attention weight on the attended pages' tokens, and the share of
the highest-weight tokens among them; -1 and out-of-row list entries are
ignored and empty requests are skipped."""
import math

import numpy as np
import pytest
import torch

import bench


def _case():
    rng = np.random.default_rng(7)
    S, d, Hq, Hkv = 2, 4, 4, 2                        # groups of 2 query heads
    lens = [5, 0, 3]                                   # pages: 3, 0, 2
    P, mp = 8, 3
    k_pool = rng.standard_normal((P, Hkv, S, d)).astype(np.float32)
    q = rng.standard_normal((3, Hq, d)).astype(np.float32)
    page_table = np.array([[4, 1, 6], [0, 0, 0], [2, 7, 3]], dtype=np.int32)
    # kept lists per (request, kv-head), padded with -1; 9 lies past every row
    sel = np.array([[[0, 2, -1], [1, -1, 9]],
                    [[0, 1, 2], [0, 1, 2]],
                    [[1, -1, -1], [0, 1, -1]]], dtype=np.int32)
    return q, k_pool, page_table, np.array(lens, dtype=np.int32), sel, S


def _direct(q, k_pool, pt, lens, sel, S, scale, m):
    Hq, Hkv = q.shape[1], k_pool.shape[1]
    G = Hq // Hkv
    mass, top = [], []
    for b, L in enumerate(lens):
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            keys = np.stack([k_pool[pt[b, t // S], g, t % S] for t in range(L)])
            z = keys.astype(np.float64) @ q[b, h].astype(np.float64) * scale
            w = np.exp(z - z.max())
            w /= w.sum()
            kept = {int(j) for j in sel[b, g] if 0 <= j < -(-L // S)}
            in_kept = np.array([t // S in kept for t in range(L)])
            mass.append(float(w[in_kept].sum()))
            best = np.argsort(-w, kind="stable")[:min(m, L)]
            top.append(float(in_kept[best].mean()))
    return mass, top


@pytest.mark.parametrize("m", [1, 2, 16])
def test_attention_recall_matches_its_definition(m):
    q, k_pool, pt, lens, sel, S = _case()
    scale = 1 / math.sqrt(q.shape[-1])
    got = bench.attention_recall(torch, torch.from_numpy(q), torch.from_numpy(k_pool),
                                 torch.from_numpy(pt), torch.from_numpy(lens),
                                 torch.from_numpy(sel), S, scale, top_m=m)
    mass, top = _direct(q, k_pool, pt, lens, sel, S, scale, m)
    assert len(mass) == 8                               # 2 requests with tokens x 4 heads
    assert got["mass_mean"] == pytest.approx(np.mean(mass), abs=1e-6)
    assert got["mass_min"] == pytest.approx(min(mass), abs=1e-6)
    assert got[f"top{m}_mean"] == pytest.approx(np.mean(top), abs=1e-6)
    assert got[f"top{m}_min"] == pytest.approx(min(top), abs=1e-6)


def test_keeping_every_page_recalls_everything():
    q, k_pool, pt, lens, sel, S = _case()
    every = np.tile(np.arange(3, dtype=np.int32), (3, 2, 1))
    got = bench.attention_recall(torch, torch.from_numpy(q), torch.from_numpy(k_pool),
                                 torch.from_numpy(pt), torch.from_numpy(lens),
                                 torch.from_numpy(every), S, 0.5)
    assert got["mass_min"] == pytest.approx(1.0, abs=1e-6)
    assert got["top16_min"] == 1.0
