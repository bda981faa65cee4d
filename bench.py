"""Benchmark of the Quest sparse decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload longchat]

A "step" is one pass of the whole hot path -- quest_estimate ->
quest_topk_sparse_decode_attn (Top-K + sparse attention + split merge) --
replayed as a HIP graph, over one LongChat-7B-shaped
layer (32 heads, 32K context, 2048-token budget, fp16).  Inputs are seeded
synthetic caches drawn on the GPU and resident in HBM before timing starts.
Consecutive steps rotate over several independent caches whose touched bytes
(metadata + selected pages) together exceed the 256 MB Infinity Cache, so
every step reads its bytes from HBM.

Prints ONE JSON line: the step time (the metric), effective GB/s on the
algorithmic bytes, the dense-baseline time and speedup, a roofline object for
the dominant kernel (HIP-event time on the launch stream), and a CPU-oracle
baseline timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = ("µs/decode step + effective HBM GB/s, 32 heads, 32K ctx, "
          "2048-token budget")


# ------------------------------------------------------------- byte model

def step_bytes(seq_lens, n_kv_heads, n_q_heads, k_pages, sel=None,
               page_size=16, d=128, s=2):
    """Algorithmic bytes of one sparse step: every page's min/max metadata,
    the valid tokens of the selected pages' K and V (once per kv-head), q,
    the fp32 output and the page-table entries read."""
    meta = kv = 0
    table = 0
    for b, L in enumerate(seq_lens):
        n = -(-L // page_size)
        meta += n_kv_heads * n * 2 * d * s
        table += n * 4
        if sel is None:          # assume the kept pages are full pages
            kv += n_kv_heads * min(k_pages, n) * page_size * 2 * d * s
        else:
            for g in range(n_kv_heads):
                for j in sel[b][g]:
                    if j >= 0:
                        v = min(page_size, L - j * page_size)
                        kv += v * 2 * d * s
    B = len(seq_lens)
    q = B * n_q_heads * d * s
    out = B * n_q_heads * d * 4
    return dict(meta=meta, kv=kv, q=q, out=out, table=table,
                total=meta + kv + q + out + table)


def dense_bytes(seq_lens, n_kv_heads, n_q_heads, page_size=16, d=128, s=2):
    kv = sum(L * n_kv_heads * 2 * d * s for L in seq_lens)
    B = len(seq_lens)
    return kv + B * n_q_heads * d * (s + 4) + sum(-(-L // page_size) * 4
                                                  for L in seq_lens)


def kv_cache_bytes(layers, heads, d, ctx, s=2):
    """K and V of every layer and head for ctx tokens."""
    return layers * 2 * heads * d * ctx * s


# ------------------------------------------------------------- GPU timing

class KernelTimer:
    """Events recorded on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def around(self, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        self.pairs.append((e0, e1))

    def mean_us(self):
        self.torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in self.pairs]
        return sum(ts) / len(ts) if ts else float("nan")


def run_gpu(args):
    import numpy as np
    import torch

    import query_aware_kv_amd as qa
    import synth

    dev = "cuda"
    if args.workload != "longchat":
        raise SystemExit(f"unknown workload {args.workload}")
    base = synth.longchat_layer_workload()
    rot = args.rotate
    insts = []
    for i in range(rot):
        wl = synth.longchat_layer_workload(seed=base.base_seed + 1000 * i)
        c = synth.draw_layer(wl, 0, dev)
        kv = qa.paged_kv(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                         wl.pool_pages(), wl.max_pages, wl.torch_dtype)
        kmin, kmax = qa.alloc_meta(kv)
        qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                                  c["page_table"], c["seq_lens"])
        c.update(kmin=kmin, kmax=kmax, kv=kv)
        insts.append(c)
    torch.cuda.synchronize()
    kv = insts[0]["kv"]
    k = base.k_pages
    sm = 1.0 / math.sqrt(128)
    steps = [qa.SparseDecodeStep(kv, k, sm) for _ in range(rot)]
    denses = [qa.DenseDecode(kv, sm) for _ in range(rot)]
    stream = torch.cuda.current_stream()

    def step_call(i):
        c = insts[i]
        steps[i](c["q"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"],
                 c["page_table"], c["seq_lens"])

    def dense_call(i):
        c = insts[i]
        denses[i](c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    for i in range(rot):                 # eager warm-up before capture
        step_call(i)
        dense_call(i)
    torch.cuda.synchronize()
    step_graphs = [capture(lambda i=i: step_call(i)) for i in range(rot)]
    dense_graphs = [capture(lambda i=i: dense_call(i)) for i in range(rot)]

    def timed(fn, n, w):
        for i in range(w):
            fn(i % rot)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            fn(i % rot)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e6

    us_step = timed(lambda i: step_graphs[i].replay(), args.steps, args.warmup)
    us_eager = timed(step_call, args.steps, args.warmup)
    us_dense = (float("nan") if args.no_dense else
                timed(lambda i: dense_graphs[i].replay(), max(20, args.steps // 4),
                      args.warmup))

    # Per-call device time: HIP events on the launch stream around replays of
    # a graph holding one launch of the call per cache (8 back to back).
    def call_us(call, reps=max(10, args.steps // rot)):
        g = capture(lambda: [call(i) for i in range(rot)])
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * rot)

    def est(i):
        c, st = insts[i], steps[i]
        qa.quest_estimate(kv, c["q"], c["kmin"], c["kmax"], c["page_table"],
                          c["seq_lens"], st.scores)

    def topk_attn(i):
        c, st = insts[i], steps[i]
        qa.quest_topk_sparse_decode_attn(
            kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"],
            c["seq_lens"], st.scores, k, sm, st.sel, st.out, st.workspace)

    us_est = call_us(est)
    us_ta = call_us(topk_attn)

    # algorithmic bytes from the selections actually made
    sels = [st.sel.cpu().numpy() for st in steps]
    lens = [int(x) for x in insts[0]["seq_lens"].cpu()]
    bstep = [step_bytes(lens, kv.num_kv_heads, kv.num_q_heads, k, sel=s)
             for s in sels]
    avg = {key: sum(b[key] for b in bstep) / len(bstep) for key in bstep[0]}
    B = len(lens)
    est_bytes = avg["meta"] + avg["q"] + avg["table"] + \
        kv.num_kv_heads * kv.max_pages_per_seq * 4 * B
    ta_bytes = avg["kv"] + avg["q"] + avg["out"] + \
        kv.num_kv_heads * (kv.max_pages_per_seq + k) * 4 * B
    calls = {"quest_estimate [estimate_kernel]": (us_est, est_bytes),
             "quest_topk_sparse_decode_attn [topk_attn_kernel + attn_merge_kernel]":
                 (us_ta, ta_bytes)}
    dom = max(calls, key=lambda c: calls[c][0])
    d_us, d_bytes = calls[dom]
    achieved = d_bytes / (d_us * 1e-6) / 1e9
    return dict(
        us_step=us_step, us_eager=us_eager, us_dense=us_dense, bytes=avg,
        calls={c: round(v[0], 3) for c, v in calls.items()},
        roofline={"bound": "hbm", "achieved": round(achieved, 1),
                  "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                  "kernel": dom, "kernel_us": round(d_us, 3),
                  "bytes_per_launch": int(d_bytes)},
        dense_bytes=dense_bytes(lens, kv.num_kv_heads, kv.num_q_heads),
        gpu=torch.cuda.get_device_name(0), insts=insts, kv=kv,
        k_pages=k, sm=sm)


# ------------------------------------------------------------- CPU oracle

def cpu_baseline(gpu, budget_s):
    """The oracle's decode step on a sample of heads of the same workload,
    single-threaded, scaled to the full 32-head step."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import quest_oracle as O

    c = gpu["insts"][0]
    heads = [0, 1, 2, 3]
    f64 = lambda t: t.cpu().to(torch.float64).numpy()
    q = f64(c["q"][:, heads])
    kp = f64(c["k_pool"][:, heads])
    vp = f64(c["v_pool"][:, heads])
    pt = c["page_table"].cpu().numpy().astype(np.int64)
    lens = c["seq_lens"].cpu().numpy().astype(np.int64)
    kmin, kmax = O.page_meta(kp, pt, lens, 16)
    reps = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            O.decode_step(q, kp, vp, kmin, kmax, pt, lens, gpu["k_pages"],
                          gpu["sm"], 16)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    per_step_us = el / reps * (gpu["kv"].num_q_heads / len(heads)) * 1e6
    return {"value": round(per_step_us, 1), "unit": "us/step", "cores": 1,
            "kind": "oracle",
            "sample": (f"{reps} oracle decode steps over {len(heads)} of 32 heads "
                       f"of one 32K-context layer (estimate + Top-K + sparse "
                       f"attention, float64, 1 thread), {el:.1f} s, scaled x"
                       f"{gpu['kv'].num_q_heads // len(heads)} to 32 heads")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="longchat")
    ap.add_argument("--rotate", type=int, default=8,
                    help="independent caches the steps cycle through")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times "
                         "(calibrates the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        a = torch.empty(args.copy_probe << 20, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe << 20}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU "
              "path (the decode step shards over (request, kv-head) units "
              "with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    g = run_gpu(args)
    us = g["us_step"]
    gbps = g["bytes"]["total"] / (us * 1e-6) / 1e9
    line = {
        "metric": METRIC, "value": round(us, 3), "unit": "us/step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) fp16 K/V/q, 4 outlier channels x8, "
                "5 planted pages per head; identity page table)",
        "config": {"workload": "longchat7b_layer_decode", "batch": 1,
                   "q_heads": 32, "kv_heads": 32, "head_dim": 128,
                   "page_size": 16, "ctx": 32768, "budget_tokens": 2048,
                   "rotating_caches": args.rotate},
        "effective_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_step": int(g["bytes"]["total"]),
        "dense_us_per_step": round(g["us_dense"], 3),
        "speedup_vs_dense": round(g["us_dense"] / us, 3),
        "dense_effective_GBps": round(g["dense_bytes"] / (g["us_dense"] * 1e-6) / 1e9, 1),
        "timing": "HIP-graph replay of the step (one graph per cache, 8 caches "
                  "rotated); eager = the same calls issued from Python",
        "eager_us_per_step": round(g["us_eager"], 3),
        "call_us": g["calls"],
        "roofline": g["roofline"],
        "gpu": g["gpu"],
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(g, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
