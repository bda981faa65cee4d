"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Every check takes the oracle as an argument ``O`` (a module or a namespace of
functions with the oracle's names) and raises AssertionError when the oracle
breaks the property.  tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py runs them on copies of the oracle with a planted
mistake and requires at least one check to fail for each.

No check re-derives a value with the oracle's own formula: they use values
worked out by hand (tests/golden), closed forms, invariants, special cases
that reduce to a library routine, and brute force on tiny inputs.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f16_values(rng, shape, scale=1.0):
    """float64 array of fp16-representable N(0, scale^2) values."""
    return (rng.standard_normal(shape) * scale).astype(np.float16).astype(np.float64)


def small_cache(rng, B=2, Hq=2, H=2, d=16, S=4, lens=(13, 9), extra_pool=3,
                permute=True):
    """A tiny paged cache with NaN in every slot no request owns."""
    npages = [-(-L // S) for L in lens]
    P = sum(npages) + extra_pool
    k_pool = np.full((P, H, S, d), np.nan)
    v_pool = np.full((P, H, S, d), np.nan)
    perm = rng.permutation(P) if permute else np.arange(P)
    mp = max(npages) + 1
    pt = np.zeros((B, mp), dtype=np.int64)
    off = 0
    for b, L in enumerate(lens):
        for j in range(npages[b]):
            p = perm[off + j]
            pt[b, j] = p
            v = min(S, L - j * S)
            k_pool[p, :, :v] = f16_values(rng, (H, v, d))
            v_pool[p, :, :v] = f16_values(rng, (H, v, d))
        off += npages[b]
    q = f16_values(rng, (B, Hq, d))
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, page_table=pt,
                seq_lens=np.array(lens), S=S)


def _valid_tokens(c, b, j, g):
    L = int(c["seq_lens"][b])
    S = c["S"]
    v = max(0, min(S, L - j * S))
    p = int(c["page_table"][b, j])
    return c["k_pool"][p, g, :v]


# ---------------------------------------------------------------- metadata

def check_meta_bounds_attained(O, seed=0):
    """kmin/kmax bound every valid key and are attained by one (which
    characterises min and max) -- Guide to Quest §1."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng)
    kmin, kmax = O.page_meta(c["k_pool"], c["page_table"], c["seq_lens"], c["S"])
    for b, L in enumerate(c["seq_lens"]):
        for j in range(-(-int(L) // c["S"])):
            p = int(c["page_table"][b, j])
            for g in range(c["k_pool"].shape[1]):
                t = _valid_tokens(c, b, j, g)
                assert np.all(kmin[p, g] <= t) and np.all(kmax[p, g] >= t)
                assert np.all((t == kmin[p, g]).any(axis=0))
                assert np.all((t == kmax[p, g]).any(axis=0))


def check_meta_single_token_page(O):
    """A page holding one token has kmin = kmax = that token."""
    rng = np.random.default_rng(1)
    c = small_cache(rng, lens=(9, 5), S=4)    # last pages hold 1 token
    kmin, kmax = O.page_meta(c["k_pool"], c["page_table"], c["seq_lens"], c["S"])
    for b in range(2):
        j = (int(c["seq_lens"][b]) - 1) // 4
        p = int(c["page_table"][b, j])
        tok = c["k_pool"][p, :, 0]
        assert np.array_equal(kmin[p], tok) and np.array_equal(kmax[p], tok)


def check_meta_signed_zero(O):
    """-0 < +0: min of {-0, +0} is -0, max is +0; all -0 -> max is -0."""
    S, d = 4, 3
    k_pool = np.full((1, 1, S, d), np.nan)
    k_pool[0, 0, 0] = [-0.0, 0.0, -0.0]
    k_pool[0, 0, 1] = [0.0, 0.0, -0.0]
    pt = np.zeros((1, 1), dtype=np.int64)
    kmin, kmax = O.page_meta(k_pool, pt, np.array([2]), S)
    assert list(np.signbit(kmin[0, 0])) == [True, False, True]
    assert list(np.signbit(kmax[0, 0])) == [False, False, True]
    assert np.all(kmin[0, 0] == 0) and np.all(kmax[0, 0] == 0)


def check_append_equals_rebuild(O, seed=2):
    """Appending tokens one at a time gives the same boxes, bit for bit
    (signed zeros included), as building them from the whole page."""
    rng = np.random.default_rng(seed)
    B, H, S, d = 2, 2, 4, 8
    lens = [11, 6]
    c = small_cache(rng, B=B, Hq=H, H=H, d=d, S=S, lens=lens)
    # sprinkle signed zeros into the keys
    for b, L in enumerate(lens):
        for j in range(-(-L // S)):
            p = c["page_table"][b, j]
            mask = rng.random((H, S, d)) < 0.15
            c["k_pool"][p][mask & ~np.isnan(c["k_pool"][p])] = 0.0
            mask = rng.random((H, S, d)) < 0.15
            c["k_pool"][p][mask & ~np.isnan(c["k_pool"][p])] = -0.0
    ref_min, ref_max = O.page_meta(c["k_pool"], c["page_table"],
                                   np.array(lens), S)
    P = c["k_pool"].shape[0]
    kp = np.full_like(c["k_pool"], np.nan)
    vp = np.full_like(c["v_pool"], np.nan)
    kmin = np.full((P, H, d), np.inf)
    kmax = np.full((P, H, d), -np.inf)
    for b, L in enumerate(lens):
        for pos in range(L):
            j, slot = divmod(pos, S)
            p = c["page_table"][b, j]
            O.append_token(kp, vp, kmin, kmax, c["page_table"], b, pos + 1,
                           c["k_pool"][p, :, slot], c["v_pool"][p, :, slot], S)
    used = sorted({int(c["page_table"][b, j]) for b, L in enumerate(lens)
                   for j in range(-(-L // S))})
    for p in used:
        assert np.array_equal(kmin[p], ref_min[p])
        assert np.array_equal(kmax[p], ref_max[p])
        assert np.array_equal(np.signbit(kmin[p]), np.signbit(ref_min[p]))
        assert np.array_equal(np.signbit(kmax[p]), np.signbit(ref_max[p]))


# ---------------------------------------------------------------- estimate

def _meta(O, c):
    return O.page_meta(c["k_pool"], c["page_table"], c["seq_lens"], c["S"])


def check_estimate_golden(O):
    """The hand-worked example (tests/golden/estimate_worked.json)."""
    g = load_golden("estimate_worked.json")
    S, L = g["page_size"], g["seq_len"]
    d = len(g["q"])
    k_pool = np.full((1, 1, S, d), np.nan)
    k_pool[0, 0, :L] = np.array(g["tokens"], dtype=np.float64)
    pt = np.zeros((1, 1), dtype=np.int64)
    kmin, kmax = O.page_meta(k_pool, pt, np.array([L]), S)
    assert np.array_equal(kmin[0, 0], g["kmin"])
    assert np.array_equal(kmax[0, 0], g["kmax"])
    q = np.array(g["q"], dtype=np.float64)[None, None, :]
    s = O.estimate(q, kmin, kmax, pt, np.array([L]), S)
    assert s[0, 0, 0] == g["bound_unscaled"]


def check_bound_ge_true_max(O, seed=3):
    """The estimate is at least the largest q.k in the page (Guide to Quest
    §2 inequality), for every query head of the group."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, Hq=4, H=2, d=32, S=8, lens=(61, 40))
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    G = 2
    for b, L in enumerate(c["seq_lens"]):
        for j in range(-(-int(L) // c["S"])):
            for g in range(2):
                t = _valid_tokens(c, b, j, g)
                true = sum(float((t @ c["q"][b, h]).max())
                           for h in range(g * G, (g + 1) * G))
                slack = 1e-12 * (np.abs(c["q"][b]).sum() * np.abs(t).max())
                assert s[b, g, j] >= true - slack


def check_bound_tight(O, seed=4):
    """Equality when every channel's extreme comes from the same token: one
    token per page, or all tokens identical."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, B=1, Hq=1, H=1, d=16, S=4, lens=(9,))
    p_last = int(c["page_table"][0, 2])        # holds one token
    p0 = int(c["page_table"][0, 0])
    c["k_pool"][p0, 0, :4] = c["k_pool"][p0, 0, 0]   # identical tokens
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    qv = c["q"][0, 0]
    for j, p in ((2, p_last), (0, p0)):
        true = float(c["k_pool"][p, 0, 0] @ qv)
        assert abs(s[0, 0, j] - true) <= 1e-12 * np.abs(qv).sum() * 8


def check_bound_closed_forms(O, seed=5):
    """q >= 0 gives q.Kmax; q <= 0 gives q.Kmin (Guide to Quest §2)."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, B=1, Hq=1, H=1, d=16, S=4, lens=(14,))
    kmin, kmax = _meta(O, c)
    n = 4
    pages = c["page_table"][0, :n]
    for sign in (+1, -1):
        q = np.abs(c["q"]) * sign
        s = O.estimate(q, kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
        ref = (kmax if sign > 0 else kmin)[pages, 0] @ q[0, 0]
        assert np.allclose(s[0, 0, :n], ref, rtol=1e-14, atol=1e-12)


def check_bound_is_box_maximum(O, seed=6):
    """The bound is the maximum of q.x over the box [Kmin, Kmax]: a linear
    function's maximum over a box sits at one of its 2^d corners (brute
    force over all corners, d = 8)."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, B=1, Hq=1, H=1, d=8, S=4, lens=(8,))
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    qv = c["q"][0, 0]
    for j in range(2):
        p = int(c["page_table"][0, j])
        best = -math.inf
        for corner in itertools.product((0, 1), repeat=8):
            x = np.where(np.array(corner) == 1, kmax[p, 0], kmin[p, 0])
            best = max(best, float(x @ qv))
        assert abs(s[0, 0, j] - best) <= 1e-12 * (np.abs(qv).sum() * 8)


def check_relu_form(O, seed=7):
    """Agrees with the U(q,p) simplification of Guide to Quest §2 (taken
    without its 1/sqrt(d) factor): relu(q).Kmax + min(q,0).Kmin."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, B=1, Hq=1, H=1, d=32, S=4, lens=(20,))
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    qv = c["q"][0, 0]
    pages = c["page_table"][0, :5]
    U = kmax[pages, 0] @ np.maximum(qv, 0) + kmin[pages, 0] @ np.minimum(qv, 0)
    assert np.allclose(s[0, 0, :5], U, rtol=1e-13, atol=1e-12)


def check_homogeneity(O, seed=8):
    """s(alpha q) = alpha s(q) for alpha > 0 (powers of two: exact)."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng)
    kmin, kmax = _meta(O, c)
    s1 = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    s4 = O.estimate(4.0 * c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    fin = np.isfinite(s1)
    assert np.array_equal(s4[fin], 4.0 * s1[fin])
    assert np.array_equal(np.isfinite(s4), fin)


def check_padding_and_indirection(O, seed=9):
    """Scores past the last page are -inf; moving pages around the pool
    (with the page table following) changes nothing."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, permute=False)
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    for b, L in enumerate(c["seq_lens"]):
        n = -(-int(L) // c["S"])
        assert np.all(np.isneginf(s[b, :, n:])) and np.all(np.isfinite(s[b, :, :n]))
    P = c["k_pool"].shape[0]
    perm = rng.permutation(P)                  # new home of page p: perm[p]
    k2 = np.empty_like(c["k_pool"])
    k2[perm] = c["k_pool"]
    pt2 = perm[c["page_table"]]
    kmin2, kmax2 = O.page_meta(k2, pt2, c["seq_lens"], c["S"])
    s2 = O.estimate(c["q"], kmin2, kmax2, pt2, c["seq_lens"], c["S"])
    assert np.array_equal(s, s2)


def check_gqa_group_sum(O, seed=10):
    """A group's score is the sum of its query heads' scores: splitting the
    group into single-head problems and adding them back gives the same."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, Hq=6, H=2, d=16)
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    G = 3
    for g in range(2):
        acc = np.zeros_like(s[:, g])
        for r in range(G):
            q1 = c["q"][:, g * G + r: g * G + r + 1]
            q_only = np.zeros((2, 2, 16))
            q_only[:, g] = q1[:, 0]
            s1 = O.estimate(q_only, kmin, kmax, c["page_table"],
                            c["seq_lens"], c["S"])
            acc = acc + s1[:, g]
        fin = np.isfinite(s[:, g])
        assert np.allclose(acc[fin], s[:, g][fin], rtol=1e-13, atol=1e-12)


# ---------------------------------------------------------------- Top-K

def _qualifies(s, S):
    """S is the Top-K under (score desc, index asc) iff every kept page beats
    every dropped one."""
    n = len(s)
    for x in S:
        for y in range(n):
            if y in S:
                continue
            if not (s[x] > s[y] or (s[x] == s[y] and x < y)):
                return False
    return True


def check_topk_golden(O):
    g = load_golden("topk_ties.json")
    s = np.array([float(x) for x in g["scores"]])
    for case in g["cases"]:
        got = O.topk_pages(s, len(s), case["k"])
        assert list(got) == case["expect"], (case, got)


def check_topk_bruteforce(O, seed=11):
    """Exhaustive search over every subset of n <= 10 pages: exactly one
    subset qualifies, and it is the one selected.  Integer scores make ties
    common."""
    rng = np.random.default_rng(seed)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 12))
        s = rng.integers(-3, 4, n).astype(np.float64)
        kk = min(k, n)
        winners = [set(S) for S in itertools.combinations(range(n), kk)
                   if _qualifies(s, set(S))]
        assert len(winners) == 1
        got = O.topk_pages(s, n, k)
        assert list(got[:kk]) == sorted(winners[0])
        assert list(got[kk:]) == [-1] * (k - kk)
        # the kept set also maximises the (exact, integer) score sum
        best = max(sum(s[list(S)]) for S in itertools.combinations(range(n), kk))
        assert sum(s[got[:kk]]) == best


def check_topk_special_cases(O):
    n = 12
    assert list(O.topk_pages(np.ones(n), n, 5)) == [0, 1, 2, 3, 4]
    inc = np.arange(n, dtype=np.float64)
    assert list(O.topk_pages(inc, n, 4)) == [8, 9, 10, 11]
    assert list(O.topk_pages(-inc, n, 4)) == [0, 1, 2, 3]
    assert list(O.topk_pages(inc, n, 20)) == list(range(n)) + [-1] * 8
    assert list(O.topk_pages(np.array([-0.0, 0.0]), 2, 1)) == [0]
    assert list(O.topk_pages(np.array([0.0, -0.0]), 2, 1)) == [0]
    # only the first n entries take part
    assert list(O.topk_pages(np.array([1.0, 2.0, 99.0]), 2, 1)) == [1]


def check_topk_library(O, seed=12):
    """Same kept set as NumPy's stable argsort of the negated scores."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, 80))
        s = np.round(rng.standard_normal(n), 1)
        kk = min(k, n)
        ref = np.sort(np.argsort(-s, kind="stable")[:kk])
        got = O.topk_pages(s, n, k)
        assert np.array_equal(got[:kk], ref)


def check_forced_golden(O):
    g = load_golden("topk_forced.json")
    s = np.array([float(x) for x in g["scores"]])
    for case in g["cases"]:
        got = O.topk_pages_forced(s, len(s), case["k"], case["sink"], case["local"])
        assert list(got) == case["expect"], (case, got)


def check_forced_bruteforce(O, seed=21):
    """Exhaustive search over every subset of n <= 10 pages: among the
    subsets of size min(k, n) that hold every forced page, exactly one has
    every kept competing page beat every dropped one, and it is selected."""
    rng = np.random.default_rng(seed)
    for trial in range(80):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, 12))
        ns = int(rng.integers(0, k + 1))
        nl = int(rng.integers(0, k - ns + 1))
        s = rng.integers(-3, 4, n).astype(np.float64)
        kk = min(k, n)
        forced = set(range(min(ns, n))) | set(range(max(0, n - nl), n)) \
            if n > k else set(range(n))
        winners = []
        for S in itertools.combinations(range(n), kk):
            S = set(S)
            if not forced <= S:
                continue
            comp = S - forced
            rest = [y for y in range(n) if y not in S]
            if all(s[x] > s[y] or (s[x] == s[y] and x < y)
                   for x in comp for y in rest):
                winners.append(S)
        assert len(winners) == 1, (n, k, ns, nl)
        got = O.topk_pages_forced(s, n, k, ns, nl)
        assert list(got[:kk]) == sorted(winners[0])
        assert list(got[kk:]) == [-1] * (k - kk)


def check_forced_special_cases(O, seed=22):
    rng = np.random.default_rng(seed)
    # no forced pages is the plain rule
    for _ in range(20):
        n = int(rng.integers(1, 200))
        k = int(rng.integers(1, 60))
        sc = np.round(rng.standard_normal(n), 1)
        assert np.array_equal(O.topk_pages_forced(sc, n, k, 0, 0),
                              O.topk_pages(sc, n, k))
    # forced pages are kept however low their scores are
    n = 20
    sc = np.arange(n, dtype=np.float64)
    sc[:2] = sc[-3:] = -np.inf
    got = O.topk_pages_forced(sc, n, 8, 2, 3)
    assert list(got) == [0, 1, 14, 15, 16, 17, 18, 19]   # 16, 15, 14 compete best
    # the whole budget forced: sinks and window only
    assert list(O.topk_pages_forced(sc, n, 5, 2, 3)) == [0, 1, 17, 18, 19]
    # the window follows the sequence's end, not the row's capacity
    assert list(O.topk_pages_forced(np.zeros(40), 30, 4, 1, 2)) == [0, 1, 28, 29]
    # a budget smaller than the forced pages is refused
    try:
        O.topk_pages_forced(sc, n, 4, 2, 3)
    except ValueError:
        pass
    else:
        raise AssertionError("n_sink + n_local > k must be refused")


# ---------------------------------------------------------------- GQA union

def check_union_golden(O):
    g = load_golden("union_worked.json")
    box = np.array(g["kmin"], dtype=np.float64)[:, None, :]      # [P=4, H=1, d=2]
    pt = np.arange(4)[None, :]
    lens = np.array([4])
    k = g["k"]

    def run(qh):
        q = np.array(qh, dtype=np.float64)[None]                 # [1, 2, 2]
        s = O.estimate_heads(q, box, box, pt, lens, 1)
        sel = np.stack([O.topk_pages(s[0, h], 4, k) for h in range(2)])[None]
        return s, O.union_pages(sel, 2), q

    s, u, q = run(g["q_heads"])
    assert np.array_equal(s[0], np.array(g["expect_bounds"], dtype=np.float64))
    assert list(u[0, 0]) == g["expect_union"]
    s_sum = O.estimate(q, box, box, pt, lens, 1)
    assert list(O.topk_pages(s_sum[0, 0], 4, k)) == g["expect_sum_rule"]
    _, u2, _ = run(g["q_heads_agree"])
    assert list(u2[0, 0]) == g["expect_union_agree"]


def check_estimate_heads_sum_and_bound(O, seed=23):
    """The heads' bounds add up to the group bound (the sum rule), and each
    head's bound is at least its true max q_h . k over the page's tokens."""
    rng = np.random.default_rng(seed)
    for G in (1, 2, 4):
        c = small_cache(rng, B=2, Hq=2 * G, H=2, d=16, S=4, lens=(13, 9))
        kmin, kmax = _meta(O, c)
        sh = O.estimate_heads(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
        sg = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
        for b in range(2):
            n = -(-int(c["seq_lens"][b]) // c["S"])
            for g in range(2):
                tot = sh[b, g * G:(g + 1) * G, :n].sum(axis=0)
                assert np.allclose(tot, sg[b, g, :n], rtol=0, atol=1e-9)
                for h in range(g * G, (g + 1) * G):
                    for j in range(n):
                        keys = _valid_tokens(c, b, j, g)
                        assert sh[b, h, j] >= (keys @ c["q"][b, h]).max() - 1e-9
            assert np.all(np.isneginf(sh[b, :, n:]))


def check_union_properties(O, seed=24):
    rng = np.random.default_rng(seed)
    for trial in range(40):
        G = int(rng.choice([1, 2, 4, 8]))
        H, B = 2, 2
        k = int(rng.integers(1, 9))
        n = int(rng.integers(1, 20))
        sel = np.stack([np.stack([O.topk_pages(rng.integers(-3, 4, n).astype(float), n, k)
                                  for _ in range(H * G)]) for _ in range(B)])
        u = O.union_pages(sel, G)
        assert u.shape == (B, H, G * k)
        for b in range(B):
            for g in range(H):
                row = [int(x) for x in u[b, g]]
                kept = [x for x in row if x >= 0]
                m = len(kept)
                assert row[m:] == [-1] * (G * k - m)          # padding at the end
                assert kept == sorted(set(kept))              # ascending, no repeats
                heads = [set(int(x) for x in sel[b, h] if x >= 0)
                         for h in range(g * G, (g + 1) * G)]
                for hs in heads:
                    assert hs <= set(kept)                    # holds every head's pages
                for x in kept:
                    assert any(x in hs for hs in heads)       # and nothing else
                assert max(len(hs) for hs in heads) <= m <= min(n, G * min(k, n))
                if G == 1:
                    assert row[:k] == [int(x) for x in sel[b, g]]


# ---------------------------------------------------------------- attention

def check_attention_golden(O):
    g = load_golden("attention_worked.json")
    S, L = g["page_size"], g["seq_len"]
    d = len(g["q"])
    kp = np.full((1, 1, S, d), np.nan)
    vp = np.full((1, 1, S, d), np.nan)
    kp[0, 0, :L] = g["keys"]
    vp[0, 0, :L] = g["values"]
    q = np.array(g["q"], dtype=np.float64)[None, None]
    pt = np.zeros((1, 1), dtype=np.int64)
    scale = math.log(3.0)
    sel = np.array([[[0]]])
    for out in (O.sparse_attention(q, kp, vp, pt, np.array([L]), sel, scale, S),
                O.dense_attention(q, kp, vp, pt, np.array([L]), scale, S)):
        assert np.allclose(out[0, 0], g["expect"], rtol=0, atol=1e-14)


def check_sparse_all_equals_dense(O, seed=13):
    """Selecting every page reproduces full attention."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, Hq=4, H=2)
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    S = c["S"]
    npages = [-(-int(L) // S) for L in c["seq_lens"]]
    k = max(npages) + 2
    sel = np.full((2, 2, k), -1)
    for b in range(2):
        sel[b, :, :npages[b]] = np.arange(npages[b])
    sp = O.sparse_attention(*args, sel, 0.25, S)
    de = O.dense_attention(*args, 0.25, S)
    assert np.allclose(sp, de, rtol=0, atol=1e-12)


def check_dense_vs_sdpa(O, seed=14):
    """Dense attention equals torch's scaled_dot_product_attention (fp64,
    CPU) on the gathered sequence."""
    import torch
    rng = np.random.default_rng(seed)
    c = small_cache(rng, Hq=4, H=2, d=16)
    out = O.dense_attention(c["q"], c["k_pool"], c["v_pool"], c["page_table"],
                            c["seq_lens"], 0.3, c["S"])
    S = c["S"]
    for b, L in enumerate(c["seq_lens"]):
        L = int(L)
        pos = np.arange(L)
        phys = c["page_table"][b, pos // S]
        for h in range(4):
            g = h // 2
            K = torch.from_numpy(c["k_pool"][phys, g, pos % S])
            V = torch.from_numpy(c["v_pool"][phys, g, pos % S])
            qq = torch.from_numpy(c["q"][b, h])[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, K[None, None], V[None, None], scale=0.3)
            assert np.allclose(out[b, h], ref[0, 0, 0].numpy(), rtol=0, atol=1e-12)


def check_attention_special_cases(O, seed=15):
    """One token -> its value; identical keys or scale 0 -> mean of V;
    a huge scale -> the value of the best-matching token."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, B=1, Hq=1, H=1, d=8, S=4, lens=(1,), extra_pool=1)
    p = int(c["page_table"][0, 0])
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    sel = np.array([[[0]]])
    assert np.array_equal(O.sparse_attention(*args, sel, 0.1, 4)[0, 0],
                          c["v_pool"][p, 0, 0])
    assert np.array_equal(O.dense_attention(*args, 0.1, 4)[0, 0],
                          c["v_pool"][p, 0, 0])
    c = small_cache(rng, B=1, Hq=1, H=1, d=8, S=4, lens=(7,), extra_pool=1)
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    sel = np.array([[[0, 1]]])
    vals = np.concatenate([c["v_pool"][c["page_table"][0, 0], 0, :4],
                           c["v_pool"][c["page_table"][0, 1], 0, :3]])
    keys = np.concatenate([c["k_pool"][c["page_table"][0, 0], 0, :4],
                           c["k_pool"][c["page_table"][0, 1], 0, :3]])
    for fn in (lambda s: O.sparse_attention(*args, sel, s, 4),
               lambda s: O.dense_attention(*args, s, 4)):
        assert np.allclose(fn(0.0)[0, 0], vals.mean(axis=0), atol=1e-14)
        best = int(np.argmax(keys @ c["q"][0, 0]))
        assert np.allclose(fn(1e4)[0, 0], vals[best], atol=1e-9)
    # identical keys
    for j in range(2):
        p = c["page_table"][0, j]
        c["k_pool"][p, 0, :] = c["k_pool"][c["page_table"][0, 0], 0, 0]
    assert np.allclose(O.sparse_attention(*args, sel, 1.0, 4)[0, 0],
                       vals.mean(axis=0), atol=1e-13)


def check_attention_restricts_to_selection(O, seed=16):
    """Sparse attention over a selection equals dense attention over a new
    cache holding only the selected pages, in any order of the selection."""
    rng = np.random.default_rng(seed)
    S, d = 4, 16
    c = small_cache(rng, B=1, Hq=2, H=1, d=d, S=S, lens=(23,))
    sel = np.array([[[5, 1, 3, -1]]])           # page 5 is the partial one
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    out = O.sparse_attention(*args, sel, 0.2, S)
    out_perm = O.sparse_attention(*args, np.array([[[3, -1, 5, 1]]]), 0.2, S)
    assert np.allclose(out, out_perm, rtol=0, atol=1e-13)
    # compact cache: pages 1, 3 (full) then 5 (3 valid tokens) -> 11 tokens
    order = [1, 3, 5]
    kp = np.full((3, 1, S, d), np.nan)
    vp = np.full((3, 1, S, d), np.nan)
    for i, j in enumerate(order):
        p = c["page_table"][0, j]
        kp[i], vp[i] = c["k_pool"][p], c["v_pool"][p]
    pt = np.array([[0, 1, 2]])
    ref = O.dense_attention(c["q"], kp, vp, pt, np.array([11]), 0.2, S)
    assert np.allclose(out, ref, rtol=0, atol=1e-13)


def check_gqa_head_mapping(O):
    """Query head h reads kv-head h // G: with V constant per kv-head the
    output of each query head is that constant."""
    S, d, G, H = 4, 8, 3, 2
    rng = np.random.default_rng(17)
    c = small_cache(rng, B=1, Hq=G * H, H=H, d=d, S=S, lens=(10,), permute=False)
    for g in range(H):
        c["v_pool"][:3, g, :, :] = np.where(np.isnan(c["v_pool"][:3, g]), np.nan,
                                            float(g + 1))
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    sel = np.tile(np.array([0, 1, 2]), (1, H, 1))
    for out in (O.sparse_attention(*args, sel, 0.3, S),
                O.dense_attention(*args, 0.3, S)):
        for h in range(G * H):
            assert np.allclose(out[0, h], h // G + 1, atol=1e-14)


def check_empty_sequence(O):
    """A request with no tokens attends to nothing: zero output, no pages."""
    rng = np.random.default_rng(18)
    c = small_cache(rng, lens=(0, 6))
    args = (c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])
    kmin, kmax = _meta(O, c)
    s = O.estimate(c["q"], kmin, kmax, c["page_table"], c["seq_lens"], c["S"])
    assert np.all(np.isneginf(s[0]))
    assert list(O.topk_pages(s[0, 0], 0, 3)) == [-1, -1, -1]
    assert np.all(O.dense_attention(*args, 0.3, c["S"])[0] == 0)
    sel = np.full((2, 2, 2), -1)
    sel[1, :, :2] = [0, 1]
    assert np.all(O.sparse_attention(*args, sel, 0.3, c["S"])[0] == 0)


def check_step_full_budget_is_dense(O, seed=19):
    """With a budget of every page the decode step is full attention
    (the short-sequence rule of Implementation Step 2 in Guide to Quest)."""
    rng = np.random.default_rng(seed)
    c = small_cache(rng, Hq=4, H=2)
    kmin, kmax = _meta(O, c)
    args = (c["q"], c["k_pool"], c["v_pool"])
    s, sel, out = O.decode_step(*args, kmin, kmax, c["page_table"],
                                c["seq_lens"], 4, 0.3, c["S"])
    de = O.dense_attention(*args, c["page_table"], c["seq_lens"], 0.3, c["S"])
    assert np.allclose(out, de, rtol=0, atol=1e-12)


def check_layer_step(O, seed=20):
    """Several appended steps: boxes equal a rebuild of the grown cache, a
    dense layer is full attention over it, and a sparse layer keeps a valid
    Top-K of its own scores (every kept page beats every dropped one)."""
    rng = np.random.default_rng(seed)
    S, d, H, G = 4, 16, 2, 2
    lens0 = [6, 11]
    c = small_cache(rng, Hq=H * G, H=H, d=d, S=S, lens=(9, 14), permute=True)
    lens = np.array(lens0)
    kp, vp = c["k_pool"].copy(), c["v_pool"].copy()
    for b, L in enumerate(lens0):               # forget what is past lens0
        for pos in range(L, int(c["seq_lens"][b])):
            j, slot = divmod(pos, S)
            kp[c["page_table"][b, j], :, slot] = np.nan
            vp[c["page_table"][b, j], :, slot] = np.nan
    kmin, kmax = O.page_meta(kp, c["page_table"], lens, S)
    for step in range(3):
        lens = lens + 1
        k_new = f16_values(rng, (2, H, d))
        v_new = f16_values(rng, (2, H, d))
        layer = 0 if step == 0 else 2
        s, sel, out = O.layer_step(layer, 2, c["q"], kp, vp, kmin, kmax,
                                   c["page_table"], lens, k_new, v_new, 2,
                                   0.3, S)
        for b in range(2):
            j, slot = divmod(int(lens[b]) - 1, S)
            p = c["page_table"][b, j]
            assert np.array_equal(kp[p, :, slot], k_new[b])
        rmin, rmax = O.page_meta(kp, c["page_table"], lens, S)
        for b, L in enumerate(lens):
            for j in range(-(-int(L) // S)):
                p = c["page_table"][b, j]
                assert np.array_equal(kmin[p], rmin[p])
                assert np.array_equal(kmax[p], rmax[p])
        if layer == 0:
            assert s is None and sel is None
            de = O.dense_attention(c["q"], kp, vp, c["page_table"], lens, 0.3, S)
            assert np.allclose(out, de, rtol=0, atol=1e-12)
        else:
            for b, L in enumerate(lens):
                n = -(-int(L) // S)
                for g in range(H):
                    kept = [int(x) for x in sel[b, g] if x >= 0]
                    assert len(kept) == min(2, n) and kept == sorted(kept)
                    assert _qualifies(s[b, g, :n], set(kept))


ALL_CHECKS = [
    check_meta_bounds_attained, check_meta_single_token_page,
    check_meta_signed_zero, check_append_equals_rebuild,
    check_estimate_golden, check_bound_ge_true_max, check_bound_tight,
    check_bound_closed_forms, check_bound_is_box_maximum, check_relu_form,
    check_homogeneity, check_padding_and_indirection, check_gqa_group_sum,
    check_topk_golden, check_topk_bruteforce, check_topk_special_cases,
    check_topk_library,
    check_forced_golden, check_forced_bruteforce, check_forced_special_cases,
    check_union_golden, check_estimate_heads_sum_and_bound, check_union_properties,
    check_attention_golden, check_sparse_all_equals_dense, check_dense_vs_sdpa,
    check_attention_special_cases, check_attention_restricts_to_selection,
    check_gqa_head_mapping, check_empty_sequence,
    check_step_full_budget_is_dense, check_layer_step,
]
