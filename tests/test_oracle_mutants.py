"""Each pin must be able to fail: plant one plausible mistake in a copy of
the oracle (on the CPU) and require that at least one pin catches it."""
import types

import numpy as np
import pytest

import pins
from oracle import quest_oracle as O


def _ns(**overrides):
    ns = types.SimpleNamespace(**{n: getattr(O, n) for n in O.__all__})
    for k, v in overrides.items():
        setattr(ns, k, v)
    return ns


# ------------------------------------------------------------- the mutants

def est_dropped_kmin(q, kmin, kmax, pt, lens, S, max_pages=None):
    return O.estimate(q, kmax, kmax, pt, lens, S, max_pages)


def est_min_instead_of_max(q, kmin, kmax, pt, lens, S, max_pages=None):
    return -O.estimate(-q, kmin, kmax, pt, lens, S, max_pages)  # sum of mins


def est_scaled(q, kmin, kmax, pt, lens, S, max_pages=None):
    return O.estimate(q, kmin, kmax, pt, lens, S, max_pages) / np.sqrt(q.shape[-1])


def est_no_indirection(q, kmin, kmax, pt, lens, S, max_pages=None):
    ident = np.tile(np.arange(pt.shape[1]), (pt.shape[0], 1))
    ident = np.minimum(ident, kmin.shape[0] - 1)
    return O.estimate(q, kmin, kmax, ident, lens, S, max_pages)


def est_first_head_only(q, kmin, kmax, pt, lens, S, max_pages=None):
    B, Hq, d = q.shape
    H = kmin.shape[1]
    G = Hq // H
    q1 = np.zeros_like(q)
    q1[:, ::G] = q[:, ::G]
    return O.estimate(q1, kmin, kmax, pt, lens, S, max_pages)


def est_swapped_operands(q, kmin, kmax, pt, lens, S, max_pages=None):
    # q.kmin paired with kmax's sign test: max(q*kmin, q*kmin reversed)
    return O.estimate(q[..., ::-1].copy(), kmin, kmax, pt, lens, S, max_pages)


def topk_ties_high(scores, n, k):
    kk = min(k, n)
    s = np.asarray(scores[:n], dtype=np.float64)
    order = np.lexsort((-np.arange(n), -s))
    out = np.full(k, -1)
    out[:kk] = np.sort(order[:kk])
    return out


def topk_descending_output(scores, n, k):
    out = O.topk_pages(scores, n, k)
    kk = min(k, n)
    out[:kk] = out[:kk][::-1]
    return out


def topk_off_by_one(scores, n, k):
    return O.topk_pages(scores, n, max(0, k - 1)).tolist() + [-1]


def topk_ignores_short_rule(scores, n, k):
    s = np.concatenate([np.asarray(scores[:n], dtype=np.float64),
                        np.full(max(0, k - n), -np.inf)])
    out = O.topk_pages(s, len(s), k)
    return out


def forced_window_shifted(scores, n, k, ns, nl):
    """local window one page too early"""
    if n <= k or nl == 0:
        return O.topk_pages_forced(scores, n, k, ns, nl)
    s = np.array(scores[:n], dtype=np.float64)
    s[n - nl - 1:n - 1] = np.inf
    s[:ns] = np.inf
    return O.topk_pages(s, n, k)


def forced_full_competition(scores, n, k, ns, nl):
    """forced pages added on top of a full k-page competition"""
    out = O.topk_pages_forced(scores, n, k, 0, 0)
    if n <= k:
        return out
    kept = set(int(x) for x in out if x >= 0) | set(range(ns)) | set(range(n - nl, n))
    kept = sorted(kept)[:k]
    return np.array(kept + [-1] * (k - len(kept)))


def forced_roles_swapped(scores, n, k, ns, nl):
    """n_sink pages taken from the end and n_local from the start"""
    return O.topk_pages_forced(scores, n, k, nl, ns)


def forced_ignored(scores, n, k, ns, nl):
    return O.topk_pages(scores, n, k)


def heads_wrong_map(q, kmin, kmax, pt, lens, S, max_pages=None):
    """query head h read against kv-head h % Hkv instead of h // G"""
    B, Hq, d = q.shape
    H = kmin.shape[1]
    G = Hq // H
    perm = np.array([(h % H) * G + h // H for h in range(Hq)])
    out = O.estimate_heads(q[:, perm], kmin, kmax, pt, lens, S, max_pages)
    inv = np.argsort(perm)
    return out[:, inv]


def heads_group_sum(q, kmin, kmax, pt, lens, S, max_pages=None):
    """every head gets its group's summed bound"""
    B, Hq, d = q.shape
    G = Hq // kmin.shape[1]
    s = O.estimate(q, kmin, kmax, pt, lens, S, max_pages)
    return np.repeat(s, G, axis=1)


def union_drops_last_head(sel, G):
    if G == 1:
        return O.union_pages(sel, G)
    B, Hq, k = sel.shape
    s2 = sel.copy()
    s2[:, G - 1::G] = -1
    return O.union_pages(s2, G)


def union_unsorted(sel, G):
    u = O.union_pages(sel, G)
    for b in range(u.shape[0]):
        for g in range(u.shape[1]):
            m = int((u[b, g] >= 0).sum())
            u[b, g, :m] = u[b, g, :m][::-1]
    return u


def union_with_repeats(sel, G):
    B, Hq, k = sel.shape
    H = Hq // G
    out = np.full((B, H, G * k), -1, dtype=np.int64)
    for b in range(B):
        for g in range(H):
            allp = sorted(int(x) for h in range(g * G, (g + 1) * G)
                          for x in sel[b, h] if x >= 0)
            out[b, g, :len(allp)] = allp
    return out


def meta_all_slots(k_pool, pt, lens, S):
    full = np.array([-(-int(L) // S) * S for L in lens])
    return O.page_meta(k_pool, pt, full, S)


def meta_plain_minmax(k_pool, pt, lens, S):
    kmin, kmax = O.page_meta(k_pool, pt, lens, S)
    return np.where(kmin == 0, 0.0, kmin), np.where(kmax == 0, 0.0, kmax)


def append_no_reset(k_pool, v_pool, kmin, kmax, pt, b, new_len, k_new, v_new, S):
    pos = new_len - 1
    j, slot = divmod(pos, S)
    p = int(pt[b, j])
    k_pool[p, :, slot] = k_new
    v_pool[p, :, slot] = v_new
    kmin[p] = np.minimum(kmin[p], k_new)
    kmax[p] = np.maximum(kmax[p], k_new)


def sparse_unmasked(q, kp, vp, pt, lens, sel, scale, S):
    full = np.array([-(-int(L) // S) * S for L in lens])
    return O.sparse_attention(q, kp, vp, pt, full, sel, scale, S)


def sparse_wrong_heads(q, kp, vp, pt, lens, sel, scale, S):
    B, Hq, d = q.shape
    H = kp.shape[1]
    out = np.zeros((B, Hq, d))
    for h in range(Hq):                 # h % H instead of h // G
        g = h % H
        qh = np.zeros((B, H, d))
        qh[:, g] = q[:, h]
        out[:, h] = O.sparse_attention(qh, kp, vp, pt, lens, sel, scale, S)[:, g]
    return out


def sparse_no_scale(q, kp, vp, pt, lens, sel, scale, S):
    return O.sparse_attention(q, kp, vp, pt, lens, sel, 1.0, S)


def dense_unnormalised(q, kp, vp, pt, lens, scale, S):
    out = O.dense_attention(q, kp, vp, pt, lens, scale, S)
    return out * 1.0001


def dense_off_by_one_token(q, kp, vp, pt, lens, scale, S):
    return O.dense_attention(q, kp, vp, pt, np.maximum(np.asarray(lens) - 1, 1)
                             * (np.asarray(lens) > 0), scale, S)


def sparse_no_max_shift(q, kp, vp, pt, lens, sel, scale, S):
    """softmax without subtracting the running maximum"""
    B, Hq, d = q.shape
    H = kp.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(lens[b])
        for h in range(Hq):
            g = h // G
            ks, vs = [], []
            for j in sel[b, g]:
                if j < 0:
                    continue
                v = max(0, min(S, L - int(j) * S))
                p = int(pt[b, int(j)])
                ks.append(kp[p, g, :v])
                vs.append(vp[p, g, :v])
            if ks:
                w = np.exp(np.concatenate(ks) @ q[b, h] * scale)
                out[b, h] = (w @ np.concatenate(vs)) / w.sum()
    return out


def dense_no_indirection(q, kp, vp, pt, lens, scale, S):
    """pool page taken to be the logical page"""
    ident = np.tile(np.arange(pt.shape[1]), (pt.shape[0], 1))
    ident = np.minimum(ident, kp.shape[0] - 1)
    return O.dense_attention(q, kp, vp, ident, lens, scale, S)


def dense_wrong_heads(q, kp, vp, pt, lens, scale, S):
    """query head h read against kv-head h % Hkv instead of h // G"""
    B, Hq, d = q.shape
    H = kp.shape[1]
    out = np.zeros((B, Hq, d))
    for h in range(Hq):
        g = h % H
        qh = np.zeros((B, H, d))
        qh[:, g] = q[:, h]
        out[:, h] = O.dense_attention(qh, kp, vp, pt, lens, scale, S)[:, g]
    return out


def append_next_slot(k_pool, v_pool, kmin, kmax, pt, b, new_len, k_new, v_new, S):
    """the token written one slot past position new_len - 1"""
    O.append_token(k_pool, v_pool, kmin, kmax, pt, b, new_len + 1, k_new, v_new, S)


def est_floor_pages(q, kmin, kmax, pt, lens, S, max_pages=None):
    """a partial last page is not scored (n = floor(L / S))"""
    full = (np.asarray(lens) // S) * S
    s = O.estimate(q, kmin, kmax, pt, full, S,
                   pt.shape[1] if max_pages is None else max_pages)
    return s


def est_group_max(q, kmin, kmax, pt, lens, S, max_pages=None):
    """a group scored by its best head instead of the sum of its heads"""
    B, Hq, d = q.shape
    H = kmin.shape[1]
    G = Hq // H
    s = O.estimate_heads(q, kmin, kmax, pt, lens, S, max_pages)
    return s.reshape(B, H, G, -1).max(axis=2)


def topk_signed_zero(scores, n, k):
    """-0 ranked below +0 (bit order instead of value order)"""
    s = np.asarray(scores[:n], dtype=np.float64).copy()
    s[(s == 0) & np.signbit(s)] = -1e-300
    return O.topk_pages(s, n, k)


def forced_zero_window_is_everything(scores, n, k, ns, nl):
    """n_local = 0 read as a window over every page (a [-0:] slice)"""
    if nl == 0 and n > k:
        return np.arange(n - k, n)  # the "window" takes the whole budget
    return O.topk_pages_forced(scores, n, k, ns, nl)


def union_keeps_padding(sel, G):
    """the -1 padding counted as a page"""
    u = O.union_pages(sel, G)
    B, H, K = u.shape
    out = np.full_like(u, -1)
    for b in range(B):
        for g in range(H):
            pages = set(int(x) for x in u[b, g] if x >= 0)
            if (sel[b, g * G:(g + 1) * G] < 0).any():
                pages.add(-1)
            srt = sorted(pages)
            out[b, g, :len(srt)] = srt
    return out


MUTANTS = {
    "estimate_dropped_kmin": dict(estimate=est_dropped_kmin),
    "estimate_min_not_max": dict(estimate=est_min_instead_of_max),
    "estimate_scaled": dict(estimate=est_scaled),
    "estimate_no_page_table": dict(estimate=est_no_indirection),
    "estimate_first_head_only": dict(estimate=est_first_head_only),
    "estimate_swapped_channels": dict(estimate=est_swapped_operands),
    "topk_ties_to_higher": dict(topk_pages=topk_ties_high),
    "topk_descending": dict(topk_pages=topk_descending_output),
    "topk_off_by_one": dict(topk_pages=topk_off_by_one),
    "topk_no_short_rule": dict(topk_pages=topk_ignores_short_rule),
    "forced_window_shifted": dict(topk_pages_forced=forced_window_shifted),
    "forced_full_competition": dict(topk_pages_forced=forced_full_competition),
    "forced_roles_swapped": dict(topk_pages_forced=forced_roles_swapped),
    "forced_ignored": dict(topk_pages_forced=forced_ignored),
    "heads_wrong_map": dict(estimate_heads=heads_wrong_map),
    "heads_group_sum": dict(estimate_heads=heads_group_sum),
    "union_drops_last_head": dict(union_pages=union_drops_last_head),
    "union_unsorted": dict(union_pages=union_unsorted),
    "union_with_repeats": dict(union_pages=union_with_repeats),
    "meta_reads_invalid_slots": dict(page_meta=meta_all_slots),
    "meta_unsigned_zero": dict(page_meta=meta_plain_minmax),
    "append_never_resets": dict(append_token=append_no_reset),
    "sparse_unmasked_tail": dict(sparse_attention=sparse_unmasked),
    "sparse_wrong_head_map": dict(sparse_attention=sparse_wrong_heads),
    "sparse_missing_scale": dict(sparse_attention=sparse_no_scale),
    "dense_unnormalised": dict(dense_attention=dense_unnormalised),
    "dense_drops_last_token": dict(dense_attention=dense_off_by_one_token),
    "sparse_no_max_shift": dict(sparse_attention=sparse_no_max_shift),
    "dense_no_page_table": dict(dense_attention=dense_no_indirection),
    "dense_wrong_head_map": dict(dense_attention=dense_wrong_heads),
    "append_next_slot": dict(append_token=append_next_slot),
    "estimate_floor_pages": dict(estimate=est_floor_pages),
    "estimate_group_max": dict(estimate=est_group_max),
    "topk_signed_zero_order": dict(topk_pages=topk_signed_zero),
    "forced_zero_window_everything": dict(topk_pages_forced=forced_zero_window_is_everything),
    "union_keeps_padding": dict(union_pages=union_keeps_padding),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    ns = _ns(**MUTANTS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(ns)
        except AssertionError:   # a crash of the mutant does not count
            caught.append(check.__name__)
    assert caught, f"no pin catches mutant {name}"
