"""Helpers for the GPU parity tests: seeded cases, oracle runs on host
copies of the same inputs, and the comparison rules (bit-exact metadata and
Top-K, 1e-4 relative scores, boundary swaps only within 1e-4 relative,
2e-3 absolute attention)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import query_aware_kv_amd as qa
import synth
from oracle import quest_oracle as O

SCORE_RTOL = 1e-4
ATTN_ATOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 host copy (fp16, bf16 and fp32 all widen exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def workload(B=1, Hq=1, Hkv=1, lens=(1024,), budget=128, dtype="f16", seed=0,
             permute=False, outliers=0, planted=0, name="case", page_size=16):
    return synth.Workload(name, B, Hq, Hkv, tuple(lens), budget, dtype,
                          page_size=page_size, outliers=outliers,
                          planted=planted, permute_pool=permute, base_seed=seed)


def draw(wl, layer=0, heads=None):
    c = synth.draw_layer(wl, layer, "cuda", heads=heads)
    c["kv"] = qa.paged_kv(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                          wl.pool_pages(), wl.max_pages, wl.torch_dtype,
                          page_size=wl.page_size)
    return c


def gpu_meta(c):
    kv = c["kv"]
    kmin, kmax = qa.alloc_meta(kv)
    kmin.fill_(float("nan"))
    kmax.fill_(float("nan"))
    qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                              c["page_table"], c["seq_lens"])
    return kmin, kmax


def used_pages(page_table: np.ndarray, lens, S=16):
    out = []
    for b, L in enumerate(lens):
        out += [int(p) for p in page_table[b, :-(-int(L) // S)]]
    return sorted(set(out))


def assert_meta_bitexact(kmin_gpu, kmax_gpu, kmin_o, kmax_o, pages, heads=None):
    dt = kmin_gpu.dtype
    idx = torch.tensor(pages, dtype=torch.long)
    hs = slice(None) if heads is None else list(heads)
    for gpu, ora, name in ((kmin_gpu, kmin_o, "kmin"), (kmax_gpu, kmax_o, "kmax")):
        g = gpu.cpu()[idx][:, hs].view(torch.int16)
        o = torch.from_numpy(ora[pages][:, hs]).to(dt).view(torch.int16)
        bad = (g != o).nonzero()
        assert bad.numel() == 0, f"{name} differs at {bad[:5].tolist()}"


def assert_scores_close(s_gpu: np.ndarray, s_ora: np.ndarray, lens, S=16):
    for b, L in enumerate(lens):
        n = -(-int(L) // S)
        g, o = s_gpu[b, :, :n], s_ora[b, :, :n]
        err = np.abs(g - o)
        tol = SCORE_RTOL * np.abs(o)
        assert np.all(err <= tol), (
            f"b={b}: worst rel err {np.max(err / np.maximum(np.abs(o), 1e-30)):.3g}")
        assert np.all(np.isneginf(s_gpu[b, :, n:])), "padding must be -inf"


def assert_valid_selection(sel_row: np.ndarray, n: int, k: int):
    kk = min(k, n)
    kept = sel_row[:kk]
    assert np.all(sel_row[kk:] == -1), "padding must be -1"
    assert np.all(kept >= 0) and np.all(kept < n), "page index out of range"
    assert np.all(np.diff(kept) > 0), "must be strictly ascending"


def assert_sets_match(sel_gpu: np.ndarray, s_ora: np.ndarray, lens, k, S=16,
                      n_sink=0, n_local=0):
    """Identical to the oracle's Top-K (on its float64 scores; with forced
    sink / local pages if given) except for swaps x in G-O, y in O-G with
    s_y - s_x <= 1e-4 max(|s_x|, |s_y|).  Returns the number of swapped
    pages."""
    swaps = 0
    B, H = sel_gpu.shape[:2]
    for b in range(B):
        n = -(-int(lens[b]) // S)
        for g in range(H):
            assert_valid_selection(sel_gpu[b, g], n, k)
            if n_sink or n_local:
                o = O.topk_pages_forced(s_ora[b, g], n, k, n_sink, n_local)
            else:
                o = O.topk_pages(s_ora[b, g], n, k)
            G_ = set(int(x) for x in sel_gpu[b, g] if x >= 0)
            O_ = set(int(x) for x in o if x >= 0)
            only_g, only_o = G_ - O_, O_ - G_
            for x in only_g:
                for y in only_o:
                    sx, sy = s_ora[b, g, x], s_ora[b, g, y]
                    assert sy - sx <= SCORE_RTOL * max(abs(sx), abs(sy)), (
                        f"b={b} g={g}: kept {x} ({sx}) over {y} ({sy})")
            swaps += len(only_g)
    return swaps


def oracle_inputs(c, heads=None):
    """Host float64 copies of the inputs (optionally only some kv-heads;
    the other heads are NaN)."""
    q = to64(c["q"])
    if heads is None:
        kp, vp = to64(c["k_pool"]), to64(c["v_pool"])
    else:
        P, H, S, d = c["k_pool"].shape
        kp = np.full((P, H, S, d), np.nan)
        vp = np.full((P, H, S, d), np.nan)
        for g in heads:
            kp[:, g] = to64(c["k_pool"][:, g])
            vp[:, g] = to64(c["v_pool"][:, g])
    return dict(q=q, k_pool=kp, v_pool=vp,
                page_table=c["page_table"].cpu().numpy().astype(np.int64),
                seq_lens=c["seq_lens"].cpu().numpy().astype(np.int64))


def run_gpu_step(c, k_pages, kmin, kmax, sm_scale, select="attention", n_sink=0,
                 n_local=0):
    step = qa.SparseDecodeStep(c["kv"], k_pages, sm_scale, select=select,
                               n_sink=n_sink, n_local=n_local)
    out = step(c["q"], c["k_pool"], c["v_pool"], kmin, kmax,
               c["page_table"], c["seq_lens"])
    torch.cuda.synchronize()
    return step.scores.cpu().numpy().astype(np.float64), \
        step.sel.cpu().numpy().astype(np.int64), out.cpu().numpy().astype(np.float64)


# Two GPU paths that attend over the same pages but split and merge them
# differently (the one-launch Top-K + attention uses 8-wave workgroups, the
# separate attention 4-wave ones) sum the same float32 terms in a different
# order: equal up to float32 rounding of sums of at most a few thousand
# terms of magnitude <= 1.
SPLIT_ORDER_TOL = 1e-5


def assert_same_up_to_split_order(a: torch.Tensor, b: torch.Tensor):
    err = float((a - b).abs().max()) if a.numel() else 0.0
    assert err <= SPLIT_ORDER_TOL, f"max |a - b| = {err:.3g}"


def assert_attention_close(out_gpu: np.ndarray, out_ora: np.ndarray, rows=None):
    if rows is not None:
        out_gpu, out_ora = out_gpu[rows], out_ora[rows]
    err = np.max(np.abs(out_gpu - out_ora)) if out_gpu.size else 0.0
    assert err <= ATTN_ATOL, f"max |out - oracle| = {err:.3g}"
    return err
