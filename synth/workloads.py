"""Seeded synthetic inputs shaped like the Quest decode workloads.

This module draws the inputs of one decode step -- the query, the paged K/V
pools, the page table and the sequence lengths -- and nothing else.  It holds
none of the method's arithmetic (no page metadata, no bound, no selection, no
attention); both the CPU oracle and the HIP path consume what it produces.

Structure of the draws (the pages fix the shapes, the recipe is ours):

* K, V and q are i.i.d. N(0, 1), drawn in fp32 and rounded once (RNE) to the
  storage dtype (fp16 or bf16).
* Outlier channels: for each (layer, kv-head), ``outliers`` channel indices
  are drawn without replacement and those channels of every K row (appended
  rows included) are multiplied by ``outlier_scale`` before rounding.
* Planted pages: for each (request, kv-head), ``planted`` distinct logical
  pages are drawn; every token in them gets the key
  ``|k0| * (cos * q_hat + sqrt(1 - cos^2) * u_perp)`` where ``q_hat`` is the
  unit (rounded) query of that head, ``u_perp`` a random unit vector
  orthogonal to it and ``|k0|`` the norm of the token's own outlier-scaled
  row.  This makes the page selection non-trivial.
* Page table: the identity over each request's span of the pool, or a seeded
  permutation of the whole pool.  Entries past a request's last page hold 0
  (a valid page id that is never read).
* Slots past a request's last valid token (the tail of its last page) and
  pool pages that no request owns are filled with NaN: callers promise
  nothing about those bytes, so kernels must never use them as values.

Random streams are keyed per unit (``unit_seed``) so any (layer, request,
kv-head) slice can be regenerated alone.  Structural choices (outlier
channels, planted page indices, ragged lengths, the pool permutation) are
drawn on the CPU and are identical on every device; the bulk N(0, 1) values
come from the generator of the device they are drawn on.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional, Sequence

import torch

HEAD_DIM = 128
PAGE_SIZE = 16

_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def unit_seed(*key) -> int:
    """Stable 63-bit seed for a tuple key (ints and strings)."""
    h = hashlib.blake2b(repr(tuple(key)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(device, *key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(unit_seed(*key))
    return g


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload.  ``seq_lens`` are the attended lengths L_b."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: tuple
    budget_tokens: int
    dtype: str = "f16"
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE
    outliers: int = 0
    outlier_scale: float = 8.0
    planted: int = 0
    planted_cos: float = 0.9
    permute_pool: bool = False
    layers: int = 1
    steps: int = 0           # decode steps that append one token each
    dense_layers: int = 0    # leading layers that run dense attention
    base_seed: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def k_pages(self) -> int:
        return self.budget_tokens // self.page_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    def final_lens(self) -> List[int]:
        return [L + self.steps for L in self.seq_lens]

    @property
    def max_pages(self) -> int:
        return max(1, max(-(-L // self.page_size) for L in self.final_lens()))

    def pool_pages(self) -> int:
        return max(1, sum(-(-L // self.page_size) for L in self.final_lens()))


# ---------------------------------------------------------------------------
# The workloads of the pages (shapes from the pages' statement of the
# problem; see the module docstring for the recipe).
# ---------------------------------------------------------------------------

def tiny_workload(seed: int = 0) -> Workload:
    """1 head, 1K context (64 pages), 8-page budget, plain N(0,1) fp16."""
    return Workload("tiny", 1, 1, 1, (1024,), 128, "f16", base_seed=seed)


def longchat_layer_workload(ctx: int = 32768, budget: int = 2048,
                            seed: int = 1) -> Workload:
    """One LongChat-7B-shaped decode layer: 32 heads, fp16, outlier
    channels and planted pages."""
    return Workload(f"longchat7b_layer_ctx{ctx}_budget{budget}", 1, 32, 32,
                    (ctx,), budget, "f16", outliers=4, planted=5,
                    base_seed=seed)


def sweep_workload(ctx: int, budget: int, seed: int = 2) -> Workload:
    return dataclasses.replace(longchat_layer_workload(ctx, budget, seed),
                               name=f"sweep_ctx{ctx}_budget{budget}")


SWEEP_CTX = (4096, 16384, 32768, 65536, 131072)
SWEEP_BUDGET = (256, 512, 1024, 2048, 4096)


def ragged_lengths(batch: int, lo: int, hi: int, seed: int) -> tuple:
    g = _gen("cpu", seed, "ragged_lens")
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (batch,),
                                               generator=g))


def ragged_batch_workload(seed: int = 3, batch: int = 32, lo: int = 8192,
                          hi: int = 32768) -> Workload:
    """32 requests x 32 heads, contexts uniform in [8K, 32K], bf16,
    pages scattered through a shared pool by a seeded permutation."""
    return Workload(f"ragged_b{batch}", batch, 32, 32,
                    ragged_lengths(batch, lo, hi, seed), 2048, "bf16",
                    permute_pool=True, base_seed=seed)


def gqa_multistep_workload(seed: int = 4, layers: int = 32, steps: int = 128,
                           ctx: int = 32768) -> Workload:
    """32 layers of 32 q-heads / 8 kv-heads, 32K start, one appended token
    per step, first two layers dense, 2048-token budget, outliers."""
    return Workload(f"gqa_l{layers}_s{steps}", 1, 32, 8, (ctx,), 2048, "f16",
                    outliers=4, layers=layers, steps=steps, dense_layers=2,
                    base_seed=seed)


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------

def page_table_for(wl: Workload) -> torch.Tensor:
    """int32 [B, max_pages]: logical page j of request b -> pool page."""
    B, mp = wl.batch, wl.max_pages
    npages = [-(-L // wl.page_size) for L in wl.final_lens()]
    P = wl.pool_pages()
    if wl.permute_pool:
        perm = torch.randperm(P, generator=_gen("cpu", wl.base_seed, "perm"))
    else:
        perm = torch.arange(P)
    pt = torch.zeros(B, mp, dtype=torch.int32)
    off = 0
    for b in range(B):
        pt[b, :npages[b]] = perm[off:off + npages[b]].to(torch.int32)
        off += npages[b]
    return pt


def outlier_channels(wl: Workload, layer: int, g: int) -> torch.Tensor:
    if wl.outliers == 0:
        return torch.zeros(0, dtype=torch.long)
    gen = _gen("cpu", wl.base_seed, "outlier", layer, g)
    return torch.randperm(wl.head_dim, generator=gen)[:wl.outliers]


def planted_pages(wl: Workload, layer: int, b: int, g: int,
                  n_pages: int) -> torch.Tensor:
    if wl.planted == 0 or n_pages == 0:
        return torch.zeros(0, dtype=torch.long)
    gen = _gen("cpu", wl.base_seed, "plant", layer, b, g)
    m = min(wl.planted, n_pages)
    return torch.sort(torch.randperm(n_pages, generator=gen)[:m]).values


def draw_query(wl: Workload, layer: int, device, step: int = -1) -> torch.Tensor:
    """q [B, Hq, d] in the storage dtype."""
    out = torch.empty(wl.batch, wl.num_q_heads, wl.head_dim,
                      dtype=wl.torch_dtype, device=device)
    for b in range(wl.batch):
        gen = _gen(device, wl.base_seed, "q", layer, step, b)
        x = torch.randn(wl.num_q_heads, wl.head_dim, generator=gen,
                        device=device, dtype=torch.float32)
        out[b] = x.to(wl.torch_dtype)
    return out


def _planted_rows(k_rows: torch.Tensor, q_hat: torch.Tensor, cos: float,
                  gen: torch.Generator) -> torch.Tensor:
    """Replace each row by |row| * (cos*q_hat + sin*u_perp)."""
    n = k_rows.shape[0]
    u = torch.randn(n, q_hat.numel(), generator=gen, device=k_rows.device,
                    dtype=torch.float32)
    u = u - (u @ q_hat)[:, None] * q_hat[None, :]
    u = u / u.norm(dim=1, keepdim=True)
    norm = k_rows.norm(dim=1, keepdim=True)
    sin = math.sqrt(1.0 - cos * cos)
    return norm * (cos * q_hat[None, :] + sin * u)


def draw_cache(wl: Workload, layer: int, device, q: torch.Tensor,
               lens: Optional[Sequence[int]] = None,
               heads: Optional[Sequence[int]] = None) -> Dict[str, torch.Tensor]:
    """K/V pools [P, Hkv, page, d] holding ``lens`` (default wl.seq_lens)
    tokens per request; everything else in the pools is NaN.

    ``q`` is the layer's query (needed only for planted pages).  ``heads``
    restricts the draw to some kv-heads (the rest stay NaN); the values of a
    drawn head do not depend on which other heads are drawn.
    """
    lens = list(wl.seq_lens if lens is None else lens)
    heads = list(range(wl.num_kv_heads) if heads is None else heads)
    P, H, S, d = wl.pool_pages(), wl.num_kv_heads, wl.page_size, wl.head_dim
    dt = wl.torch_dtype
    pt = page_table_for(wl)
    k_pool = torch.full((P, H, S, d), float("nan"), dtype=dt, device=device)
    v_pool = torch.full((P, H, S, d), float("nan"), dtype=dt, device=device)
    for b in range(wl.batch):
        L = lens[b]
        n = -(-L // S)
        if n == 0:
            continue
        pages = pt[b, :n].to(torch.long).to(device)
        for g in heads:
            gk = _gen(device, wl.base_seed, "k", layer, b, g)
            gv = _gen(device, wl.base_seed, "v", layer, b, g)
            k = torch.randn(n * S, d, generator=gk, device=device,
                            dtype=torch.float32)
            v = torch.randn(n * S, d, generator=gv, device=device,
                            dtype=torch.float32)
            ch = outlier_channels(wl, layer, g).to(device)
            if ch.numel():
                k[:, ch] *= wl.outlier_scale
            plant = planted_pages(wl, layer, b, g, L // S)  # full pages only
            if plant.numel():
                h = g * wl.group
                q_hat = q[b, h].to(torch.float32)
                q_hat = q_hat / q_hat.norm()
                gp = _gen(device, wl.base_seed, "plant_u", layer, b, g)
                rows = (plant.to(device)[:, None] * S +
                        torch.arange(S, device=device)[None, :]).reshape(-1)
                k[rows] = _planted_rows(k[rows], q_hat, wl.planted_cos, gp)
            k = k.to(dt)
            v = v.to(dt)
            k[L:] = float("nan")
            v[L:] = float("nan")
            k_pool[pages, g] = k.view(n, S, d)
            v_pool[pages, g] = v.view(n, S, d)
    return {"k_pool": k_pool, "v_pool": v_pool,
            "page_table": pt.to(device),
            "seq_lens": torch.tensor(lens, dtype=torch.int32, device=device)}


def draw_append_token(wl: Workload, layer: int, step: int, device):
    """The K/V rows one decode step appends at ``layer``: [B, Hkv, d] each
    (K with the layer's outlier channels applied)."""
    B, H, d = wl.batch, wl.num_kv_heads, wl.head_dim
    k = torch.empty(B, H, d, dtype=wl.torch_dtype, device=device)
    v = torch.empty(B, H, d, dtype=wl.torch_dtype, device=device)
    for b in range(B):
        gk = _gen(device, wl.base_seed, "k_new", layer, step, b)
        gv = _gen(device, wl.base_seed, "v_new", layer, step, b)
        kf = torch.randn(H, d, generator=gk, device=device, dtype=torch.float32)
        vf = torch.randn(H, d, generator=gv, device=device, dtype=torch.float32)
        for g in range(H):
            ch = outlier_channels(wl, layer, g).to(device)
            if ch.numel():
                kf[g, ch] *= wl.outlier_scale
        k[b] = kf.to(wl.torch_dtype)
        v[b] = vf.to(wl.torch_dtype)
    return k, v


def draw_layer(wl: Workload, layer: int, device, step: int = -1,
               heads: Optional[Sequence[int]] = None) -> Dict[str, torch.Tensor]:
    """Query + cache of one layer at its starting lengths."""
    q = draw_query(wl, layer, device, step=step)
    out = draw_cache(wl, layer, device, q, heads=heads)
    out["q"] = q
    return out
