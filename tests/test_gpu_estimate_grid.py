"""The bound estimate's work mappings against the oracle ("Guide to Quest",
§2 upper-bound inequality; §1 boxes for the append mode).

The kernel maps 16-lane rows to (kv-head, 4-page block) pairs in several
ways, chosen on the host from the geometry: workgroups of 8 or 4 waves on
four consecutive kv-heads when the kv-heads come in fours (else 16 rows of
consecutive kv-heads), and, on big grids, rows that walk several blocks with
a stride rounded down to the workgroup's waves.  Each case below names the
mapping it reaches; the boxes are random (kmin <= kmax) in a small pool that
requests share (page-table entries repeat, as with shared prefixes), so the
grids are large while the inputs stay small.
"""
import numpy as np
import pytest
import torch

import query_aware_kv_amd as qa
from oracle import quest_oracle as O

import gpu_cases as C

pytestmark = pytest.mark.gpu

S = 16
TARGET_ROWS = 196608   # the estimate's grid target (16-lane rows per launch)


def mapping(B, Hkv, mp):
    """(kv-head quads, waves per workgroup, rows per head) the launch picks."""
    bph = -(-mp // 4)
    rph = max(1, min(TARGET_ROWS // (Hkv * B), bph))
    quads = Hkv // 4 if Hkv % 4 == 0 else 0
    waves = 8
    if quads and (rph <= 4 or quads * -(-rph // 8) * B < 256):
        waves = 4
    if quads and rph < bph and rph >= waves:
        rph -= rph % waves
    return quads, waves, rph, bph


CASES = {
    # name: (B, Hq, Hkv, max_pages, pool pages, dtype)
    # 8 waves on kv-head quads; rows walk 2 blocks, stride 61 -> 56
    "quads8_stride": (400, 32, 8, 300, 3000, "f16"),
    # the same in bf16 with 3 blocks per row (stride 491 -> 488)
    "quads8_stride_bf16": (100, 4, 4, 5000, 3000, "bf16"),
    # 4 waves: 8 rows of 2056 pages (130 workgroups at 8 waves)
    "quads4_gqa_layer": (1, 32, 8, 2056, 2056, "f16"),
    # 8 waves, one block per row, a partial last workgroup (514 = 64 * 8 + 2)
    "quads8_one_block": (1, 32, 32, 2056, 2056, "f16"),
    # rows of at most 3 blocks: 4 waves, 2000 workgroup rows
    "quads4_short": (2000, 4, 4, 10, 2500, "f16"),
    # 3 kv-head quads
    "quads8_three": (7, 24, 12, 1500, 2000, "bf16"),
    # 3 kv-heads: 16 rows of consecutive kv-heads per workgroup
    "rows16": (5, 6, 3, 700, 800, "f16"),
}


def make_case(name, seed=0, unique_last=False):
    B, Hq, Hkv, mp, P, dt = CASES[name]
    rng = np.random.default_rng(seed)
    tdt = torch.float16 if dt == "f16" else torch.bfloat16
    a = rng.standard_normal((P, Hkv, 128)).astype(np.float32)
    b = rng.standard_normal((P, Hkv, 128)).astype(np.float32)
    kmin = torch.from_numpy(np.minimum(a, b)).to(tdt)
    kmax = torch.from_numpy(np.maximum(a, b)).to(tdt)
    # lengths: empty, one token, page edges, full rows and random ones (a
    # few full or nearly full rows for small batches)
    if B >= 8:
        edge = [0, 1, S, S + 1, mp * S, mp * S - 1]
        lens = [edge[i] if i < len(edge) else int(rng.integers(1, mp * S + 1))
                for i in range(B)]
    else:
        lens = [max(1, mp * S - 7 * i) for i in range(B)]
    lens = np.array(lens, dtype=np.int32)
    pt = rng.integers(0, P, size=(B, mp)).astype(np.int32)
    if unique_last:
        # every request appends into a page of its own
        assert P >= B
        others = rng.integers(B, P, size=(B, mp)).astype(np.int32) if P > B else pt
        pt = others
        for r in range(B):
            if lens[r] > 0:
                pt[r, (lens[r] - 1) // S] = r
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32)).to(tdt)
    kv = qa.paged_kv(B, Hq, Hkv, P, mp, tdt)
    C.say(f"[case] estimate grid {name} B={B} Hq={Hq} Hkv={Hkv} mp={mp} P={P} {dt} "
          f"mapping(quads, waves, rows/head, blocks/head)={mapping(B, Hkv, mp)}")
    return kv, q, kmin, kmax, pt, lens


@pytest.mark.parametrize("name", sorted(CASES))
def test_estimate_grid_against_oracle(name):
    kv, q, kmin, kmax, pt, lens = make_case(name)
    scores = torch.full((kv.batch, kv.num_kv_heads, kv.max_pages_per_seq), 12345.0,
                        device="cuda")
    qa.quest_estimate(kv, q.cuda(), kmin.cuda(), kmax.cuda(), torch.from_numpy(pt).cuda(),
                      torch.from_numpy(lens).cuda(), scores)
    torch.cuda.synchronize()
    s_ora = O.estimate(C.to64(q), C.to64(kmin), C.to64(kmax), pt, lens, S,
                       kv.max_pages_per_seq)
    C.assert_scores_close(scores.cpu().numpy().astype(np.float64), s_ora, lens)


@pytest.mark.parametrize("name", ["quads8_stride", "quads8_three", "rows16"])
def test_estimate_heads_grid_against_oracle(name):
    kv, q, kmin, kmax, pt, lens = make_case(name, seed=1)
    scores = torch.full((kv.batch, kv.num_q_heads, kv.max_pages_per_seq), 12345.0,
                        device="cuda")
    qa.quest_estimate_heads(kv, q.cuda(), kmin.cuda(), kmax.cuda(),
                            torch.from_numpy(pt).cuda(), torch.from_numpy(lens).cuda(),
                            scores)
    torch.cuda.synchronize()
    s_ora = O.estimate_heads(C.to64(q), C.to64(kmin), C.to64(kmax), pt, lens, S,
                             kv.max_pages_per_seq)
    C.assert_scores_close(scores.cpu().numpy().astype(np.float64), s_ora, lens)


@pytest.mark.parametrize("name", ["quads8_stride", "quads4_short", "rows16"])
def test_append_estimate_grid_against_oracle(name):
    """The appended token lands in the block of the row that owns it, also
    when rows walk several blocks with a rounded stride."""
    kv, q, kmin, kmax, pt, lens = make_case(name, seed=2, unique_last=True)
    B, Hkv, P = kv.batch, kv.num_kv_heads, kv.num_pool_pages
    tdt = kmin.dtype
    rng = np.random.default_rng(3)
    k_new = torch.from_numpy(rng.standard_normal((B, Hkv, 128)).astype(np.float32)).to(tdt)
    v_new = torch.from_numpy(rng.standard_normal((B, Hkv, 128)).astype(np.float32)).to(tdt)
    kp = torch.zeros(P, Hkv, S, 128, dtype=tdt, device="cuda")
    vp = torch.zeros_like(kp)
    g_min, g_max = kmin.cuda(), kmax.cuda()
    scores = torch.full((B, Hkv, kv.max_pages_per_seq), 12345.0, device="cuda")
    qa.quest_append_estimate(kv, kp, vp, g_min, g_max, torch.from_numpy(pt).cuda(),
                             torch.from_numpy(lens).cuda(), k_new.cuda(), v_new.cuda(),
                             q.cuda(), scores)
    torch.cuda.synchronize()
    # the oracle: append each request's token (L = 0 requests append nothing),
    # then bound every page
    o_min, o_max = C.to64(kmin), C.to64(kmax)
    o_kp = np.zeros((P, Hkv, S, 128))
    o_vp = np.zeros_like(o_kp)
    kn, vn = C.to64(k_new), C.to64(v_new)
    touched = []
    for r in range(B):
        if lens[r] > 0:
            O.append_token(o_kp, o_vp, o_min, o_max, pt, r, int(lens[r]), kn[r], vn[r], S)
            touched.append((r, int(pt[r, (lens[r] - 1) // S]), (int(lens[r]) - 1) % S))
    s_ora = O.estimate(C.to64(q), o_min, o_max, pt, lens, S, kv.max_pages_per_seq)
    C.assert_scores_close(scores.cpu().numpy().astype(np.float64), s_ora, lens)
    pages = sorted({p for _, p, _ in touched})
    C.assert_meta_bitexact(g_min, g_max, o_min, o_max, pages)
    kp_h, vp_h = C.to64(kp), C.to64(vp)
    for r, p, slot in touched:
        assert np.array_equal(kp_h[p, :, slot], kn[r]) and np.array_equal(vp_h[p, :, slot], vn[r])
