"""CPU oracle for Quest's decode step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU
baseline leg may import this module.  The product path (the HIP library and
its Python binding) never does: it has no CPU fallback.

Plain NumPy in float64, written from the pages' equations, one function per
step, no blocking, fusion or reordering beyond what the definitions state.
All array inputs are float64 holding values exactly representable in the
storage dtype (fp16/bf16 values are exact in float64), so every product of two
inputs is exact here and only the sums round (at float64 precision).

Sources (page title, section / equation):
  [G]  "Guide to Quest: Query-Aware KV Cache Sparsity for LLMs"
       §1 "Offline Min-Max Key Vector Bounding Boxes" (min/max equation),
       §2 "Fast Query-Aware Logit Upper-Bound Estimation" (logit equation,
          the upper-bound inequality, the U(q,p) simplification),
       §3 "Top-K Page Selection and Sparse FlashAttention Dispatch",
       "The Memory Bandwidth Bottleneck of Long-Context Decoding"
          (the softmax attention equation),
       "Implementation: PyTorch Reference Kernel", Steps 1-3 (the page pool
          layout, the short-sequence rule, the gather-then-attend structure).
  [Q]  "Quest: Query-Aware Sparsity for Efficient Long-Context LLM
       Inference" (paper summary), "Summary" and "Key points".

Readings taken where the pages are silent or disagree (each is also listed
with its reason in the design notes):
  * the estimate is the unscaled max-form sum (no 1/sqrt(d));
  * a GQA group's page score is the sum of its query heads' estimates;
    query head h belongs to kv-head h // G;
  * the alternative group rule ("Best Practices" 2: per-head bounds, then the
    union of the heads' Top-K pages) is ``estimate_heads`` + a per-head
    selection + ``union_pages``: every query head of the group attends the
    union, which holds between min(k, n) and G * min(k, n) pages;
  * ties in the Top-K go to the lower page index, and scores compare as
    numbers (-0 == +0); the selection is returned in ascending page order,
    padded with -1;
  * no forced sink/local pages in the plain selection; ``topk_pages_forced``
    is the variant with them: the caller keeps n_sink + n_local <= k, so the
    result has exactly min(k, n) pages, and n_local = 0 means no window;
  * metadata and attention cover only a page's valid tokens
    (t < min(page_size, L - j*page_size));
  * min/max order signed zeros as -0 < +0 (IEEE 754-2019 minimum/maximum);
  * attention output is float64 here (the device returns fp32);
  * an empty sequence attends to nothing and yields a zero vector.

Parity pins: every function here is pinned by CPU tests against properties
the pages and mathematics fix (see tests/test_oracle_pins.py); none is
"parity unpinned".
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

__all__ = [
    "page_valid_tokens", "page_meta", "append_token", "estimate",
    "estimate_heads", "topk_pages", "topk_pages_forced", "union_pages",
    "sparse_attention", "dense_attention", "decode_step", "layer_step",
]


def page_valid_tokens(seq_len: int, j: int, page_size: int) -> int:
    """Valid tokens in logical page j of a sequence of ``seq_len`` tokens."""
    return int(max(0, min(page_size, seq_len - j * page_size)))


def _min_signed(x: np.ndarray, axis: int) -> np.ndarray:
    """Minimum along ``axis`` with -0 < +0."""
    m = x.min(axis=axis)
    neg_zero = ((x == 0) & np.signbit(x)).any(axis=axis)
    return np.where((m == 0) & neg_zero, -0.0, np.where(m == 0, 0.0, m))


def _max_signed(x: np.ndarray, axis: int) -> np.ndarray:
    """Maximum along ``axis`` with -0 < +0."""
    m = x.max(axis=axis)
    pos_zero = ((x == 0) & ~np.signbit(x)).any(axis=axis)
    return np.where((m == 0) & pos_zero, 0.0, np.where(m == 0, -0.0, m))


def page_meta(k_pool: np.ndarray, page_table: np.ndarray,
              seq_lens: np.ndarray, page_size: int):
    """Per-page, per-channel min/max of the Key vectors.

    [G] §1, min/max equation: Kmin^(p) = min_t K_{p,t}, Kmax^(p) = max_t K_{p,t},
    elementwise over the page's tokens (here: its valid tokens).

    k_pool: [P, Hkv, page_size, d].  Returns (kmin, kmax), each [P, Hkv, d];
    pages that no request uses hold NaN.
    """
    P, H, S, d = k_pool.shape
    assert S == page_size
    kmin = np.full((P, H, d), np.nan)
    kmax = np.full((P, H, d), np.nan)
    for b in range(page_table.shape[0]):
        L = int(seq_lens[b])
        for j in range(-(-L // page_size)):
            v = page_valid_tokens(L, j, page_size)
            p = int(page_table[b, j])
            tokens = k_pool[p, :, :v, :]          # [H, v, d]
            kmin[p] = _min_signed(tokens, axis=1)
            kmax[p] = _max_signed(tokens, axis=1)
    return kmin, kmax


def append_token(k_pool, v_pool, kmin, kmax, page_table, b: int,
                 new_len: int, k_new: np.ndarray, v_new: np.ndarray,
                 page_size: int) -> None:
    """Write one token (position new_len-1) of request b and fold it into its
    page's min/max, in place.

    [G] §1 builds a page's box once, as the page is formed, whether by the
    prompt or by generated tokens.  With one token appended per decode step
    the page forms one token at a time: a token in slot 0 starts a new box
    (kmin = kmax = k), any other slot widens the existing one.
    k_new, v_new: [Hkv, d].
    """
    pos = new_len - 1
    j, slot = divmod(pos, page_size)
    p = int(page_table[b, j])
    k_pool[p, :, slot, :] = k_new
    v_pool[p, :, slot, :] = v_new
    if slot == 0:
        kmin[p] = k_new
        kmax[p] = k_new
    else:
        kmin[p] = _min_signed(np.stack([kmin[p], k_new]), axis=0)
        kmax[p] = _max_signed(np.stack([kmax[p], k_new]), axis=0)


def estimate(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray,
             page_table: np.ndarray, seq_lens: np.ndarray,
             page_size: int, max_pages: Optional[int] = None) -> np.ndarray:
    """Query-aware upper bound of every page, per (request, kv-head).

    [G] §2, upper-bound inequality:
        max_t q.K_{p,t} <= sum_i max(q_i * Kmin_i, q_i * Kmax_i).
    Unscaled (no 1/sqrt(d)); a GQA group sums its query heads' bounds.

    q: [B, Hq, d].  Returns float64 [B, Hkv, max_pages], -inf past n_b.
    """
    B, Hq, d = q.shape
    H = kmin.shape[1]
    G = Hq // H
    mp = page_table.shape[1] if max_pages is None else max_pages
    s = np.full((B, H, mp), -np.inf)
    for b in range(B):
        n = -(-int(seq_lens[b]) // page_size)
        if n == 0:
            continue
        pages = page_table[b, :n].astype(np.int64)
        for g in range(H):
            lo = kmin[pages, g, :]                 # [n, d]
            hi = kmax[pages, g, :]
            total = np.zeros(n)
            for h in range(g * G, (g + 1) * G):
                qh = q[b, h, :]                    # [d]
                total += np.maximum(qh * lo, qh * hi).sum(axis=1)
            s[b, g, :n] = total
    return s


def estimate_heads(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray,
                   page_table: np.ndarray, seq_lens: np.ndarray,
                   page_size: int, max_pages: Optional[int] = None) -> np.ndarray:
    """The same upper bound for every QUERY head separately.

    [G] §2 upper-bound inequality for query head h against the box of its
    kv-head h // G; [G] Best Practices 2 computes these per-head bounds
    before taking the union of the heads' Top-K pages.

    q: [B, Hq, d].  Returns float64 [B, Hq, max_pages], -inf past n_b.
    """
    B, Hq, d = q.shape
    H = kmin.shape[1]
    G = Hq // H
    mp = page_table.shape[1] if max_pages is None else max_pages
    s = np.full((B, Hq, mp), -np.inf)
    for b in range(B):
        n = -(-int(seq_lens[b]) // page_size)
        if n == 0:
            continue
        pages = page_table[b, :n].astype(np.int64)
        for h in range(Hq):
            lo = kmin[pages, h // G, :]            # [n, d]
            hi = kmax[pages, h // G, :]
            qh = q[b, h, :]
            s[b, h, :n] = np.maximum(qh * lo, qh * hi).sum(axis=1)
    return s


def union_pages(sel_heads: np.ndarray, group: int) -> np.ndarray:
    """Union of the query heads' page selections, per kv-head.

    [G] Best Practices 2: the group loads the union of its heads' Top-K
    pages once, and every head of the group attends all of them.
    sel_heads: [B, Hq, k] per-head lists (-1 = unused), Hq = Hkv * group.
    Returns int64 [B, Hkv, group * k]: the union ascending, then -1s.
    """
    B, Hq, k = sel_heads.shape
    H = Hq // group
    out = np.full((B, H, group * k), -1, dtype=np.int64)
    for b in range(B):
        for g in range(H):
            pages = set()
            for h in range(g * group, (g + 1) * group):
                pages.update(int(x) for x in sel_heads[b, h] if x >= 0)
            u = sorted(pages)
            out[b, g, :len(u)] = u
    return out


def topk_pages(scores: np.ndarray, n_pages: int, k: int) -> np.ndarray:
    """Top-K page selection for one (request, kv-head) row.

    [G] §3: keep the K highest-bound pages; [G] Step 2: a sequence with no
    more pages than the budget keeps all of them.  Ties go to the lower index.
    Returns int64 [k]: the kept logical page indices ascending, then -1s.
    """
    kk = min(k, n_pages)
    s = np.asarray(scores[:n_pages], dtype=np.float64)
    idx = np.arange(n_pages)
    order = np.lexsort((idx, -s))                  # score desc, index asc
    chosen = np.sort(order[:kk])
    out = np.full(k, -1, dtype=np.int64)
    out[:kk] = chosen
    return out


def topk_pages_forced(scores: np.ndarray, n_pages: int, k: int, n_sink: int,
                      n_local: int) -> np.ndarray:
    """Top-K with mandatory sink and local-window pages, one row.

    [G] §3: the first pages (attention sinks) and the most recent pages
    (the local window) are always kept; the remaining budget is filled by
    the highest bounds among the other pages.  [G] Step 2: a sequence with
    no more pages than the budget keeps all of them.  Requires
    0 <= n_sink, 0 <= n_local, n_sink + n_local <= k; n_local = 0 is no
    window.  Ties among the competing pages go to the lower index.
    Returns int64 [k]: kept logical pages ascending, then -1s.
    """
    if n_sink < 0 or n_local < 0 or n_sink + n_local > k:
        raise ValueError("need 0 <= n_sink, n_local and n_sink + n_local <= k")
    if n_pages <= k:
        return topk_pages(scores, n_pages, k)
    # n_pages > k >= n_sink + n_local, so the two forced ranges are disjoint
    forced = set(range(n_sink)) | set(range(n_pages - n_local, n_pages))
    cand = np.array([j for j in range(n_pages) if j not in forced], dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)[cand]
    order = np.lexsort((cand, -s))                 # score desc, index asc
    competing = cand[order[:k - len(forced)]]
    kept = np.sort(np.concatenate([np.array(sorted(forced), dtype=np.int64),
                                   competing]))
    out = np.full(k, -1, dtype=np.int64)
    out[:len(kept)] = kept
    return out


def _softmax_weighted_sum(z: np.ndarray, values: np.ndarray) -> np.ndarray:
    """sum_t softmax(z)_t * values_t  (max-subtracted for range only)."""
    w = np.exp(z - z.max())
    return (w[:, None] * values).sum(axis=0) / w.sum()


def sparse_attention(q, k_pool, v_pool, page_table, seq_lens, sel,
                     sm_scale: float, page_size: int) -> np.ndarray:
    """Exact softmax attention over only the selected pages' valid tokens.

    [Q] Summary: exact attention over the Top-K pages; [G] §3 and Step 3:
    gather the selected pages' K/V, then softmax(q K^T * scale) V.
    sel: [B, Hkv, k] logical page indices (-1 = unused).  Query head h reads
    kv-head h // G.  Returns float64 [B, Hq, d].
    """
    B, Hq, d = q.shape
    H = k_pool.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            g = h // G
            keys: List[np.ndarray] = []
            vals: List[np.ndarray] = []
            for j in sel[b, g]:
                if j < 0:
                    continue
                v = page_valid_tokens(L, int(j), page_size)
                p = int(page_table[b, int(j)])
                keys.append(k_pool[p, g, :v, :])
                vals.append(v_pool[p, g, :v, :])
            if not keys:
                continue
            K = np.concatenate(keys)
            V = np.concatenate(vals)
            z = (K @ q[b, h]) * sm_scale
            out[b, h] = _softmax_weighted_sum(z, V)
    return out


def dense_attention(q, k_pool, v_pool, page_table, seq_lens,
                    sm_scale: float, page_size: int) -> np.ndarray:
    """Textbook decode attention over every token 0..L-1.

    "The Memory Bandwidth Bottleneck of Long-Context Decoding" in [G]:
    Attention(Q, K, V) = softmax(Q K^T / sqrt(d)) V.  Written independently
    of ``sparse_attention``: tokens are gathered by sequence position.
    """
    B, Hq, d = q.shape
    H = k_pool.shape[1]
    G = Hq // H
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        phys = page_table[b, pos // page_size].astype(np.int64)
        slot = pos % page_size
        for h in range(Hq):
            g = h // G
            K = k_pool[phys, g, slot, :]           # [L, d]
            V = v_pool[phys, g, slot, :]
            logits = K @ q[b, h] * sm_scale
            w = np.exp(logits - logits.max())
            out[b, h] = (w @ V) / w.sum()
    return out


def decode_step(q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                k_pages: int, sm_scale: float, page_size: int):
    """One sparse decode step: estimate -> Top-K -> sparse attention.

    Returns (scores float64 [B, Hkv, max_pages], sel int64 [B, Hkv, k],
    out float64 [B, Hq, d]).
    """
    s = estimate(q, kmin, kmax, page_table, seq_lens, page_size)
    B, H = s.shape[:2]
    sel = np.full((B, H, k_pages), -1, dtype=np.int64)
    for b in range(B):
        n = -(-int(seq_lens[b]) // page_size)
        for g in range(H):
            sel[b, g] = topk_pages(s[b, g], n, k_pages)
    out = sparse_attention(q, k_pool, v_pool, page_table, seq_lens, sel,
                           sm_scale, page_size)
    return s, sel, out


def layer_step(layer: int, dense_layers: int, q, k_pool, v_pool, kmin, kmax,
               page_table, seq_lens, k_new, v_new, k_pages: int,
               sm_scale: float, page_size: int):
    """One layer of one decode step with an appended token, in place.

    Each request first appends its new token (position seq_lens[b]-1;
    ``seq_lens`` are the lengths after the append) and folds it into its
    page's box.  The leading ``dense_layers`` layers then attend densely --
    the Quest paper summary ("Key points") reports the skipping outside the
    first two layers -- and every later layer runs the sparse step.
    Returns (scores | None, sel | None, out).
    """
    for b in range(q.shape[0]):
        append_token(k_pool, v_pool, kmin, kmax, page_table, b,
                     int(seq_lens[b]), k_new[b], v_new[b], page_size)
    if layer < dense_layers:
        return None, None, dense_attention(q, k_pool, v_pool, page_table,
                                           seq_lens, sm_scale, page_size)
    return decode_step(q, k_pool, v_pool, kmin, kmax, page_table, seq_lens,
                       k_pages, sm_scale, page_size)
