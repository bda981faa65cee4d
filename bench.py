"""Benchmark of the Quest sparse decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Workloads (each prints ONE JSON line):

* ``longchat`` (default, the headline): one LongChat-7B-shaped layer -- 32
  heads, 32K context, 2048-token budget, fp16.  A "step" is one pass of the
  whole hot path: quest_estimate -> quest_topk_sparse_decode_attn (Top-K +
  sparse attention + split merge).  Consecutive steps rotate over 16
  independent caches whose touched bytes (metadata + selected pages, 1 GiB
  per pass) are four times the 256 MB Infinity Cache, so every step reads
  its bytes from HBM.  The value is the mean over >= 100 steps of one HIP
  graph holding a step on each cache, replayed back to back (HIP events
  around each replay; percentiles over the replays).  The same line carries
  the ragged batch, the 32-layer GQA step and two sweep points under
  ``extra`` (``--no-extra`` skips them).
* ``gqa_multistep``: 32 layers of 32 q-heads / 8 kv-heads; every step
  appends one token per layer, runs dense attention on layers 0-1
  (quest_update_page_meta in append mode, then quest_decode_attn) and the
  sparse step on layers 2-31 (quest_append_estimate, then
  quest_topk_sparse_decode_attn).  A step
  is all 32 layers; the timed steps walk the 128 appends in order.
* ``ragged``: 32 requests x 32 heads, contexts uniform in [8K, 32K], bf16,
  pages scattered through a shared pool.
* ``sweep``: the longchat layer over contexts 4K..128K x budgets 256..4096
  tokens (one line holding every point).
* ``gqa_union``: one 32/8-head GQA layer at 32K, the group-sum selection
  against per-head selection + union ("Guide to Quest", Best Practices 2):
  time, bytes and pages kept per kv-head for each rule.
* ``page32``: 16- against 32-token pages at 32K and 128K (same token
  budget), and the one-shot prefill metadata build against writing K.
* ``host_kv``: the longchat layer with K/V in pinned host memory (metadata
  in HBM): only the kept pages cross the host link; its roofline is the
  link's measured read ceiling.
* ``head_groups``: the longchat layer split into 1, 2 or 4 head groups whose
  chains run one after another or as parallel branches of one HIP graph.

Inputs are seeded synthetic tensors drawn on the GPU and resident in HBM
before timing starts.  The line carries the step time (the metric),
effective GB/s on the algorithmic bytes, the dense-baseline time and
speedup, the measured stream-read ceiling, a roofline object for the
dominant kernel (each kernel of the step timed alone, HIP events on the
launch stream, algorithmic bytes of the step's byte model with the score,
selection and partial round trips listed apart) and, for the headline, a
CPU-oracle baseline timed on a bounded sample of the same workload (one
thread, and every kv-head over one process per host core).

    python bench.py --pmc-summary DIR
    python bench.py --trace-summary DIR
    python bench.py --counter-table DIR

turn rocprofv3 CSV output into the summaries kept under profiles/: the
calibrated HBM traffic per kernel from FETCH_SIZE / WRITE_SIZE runs
(DIR/fetch, DIR/write, and DIR/cfetch, DIR/cwrite over ``--copy-probe``),
recorded with a digest of each kernel's sources and read back as the
``roofline.traffic`` of the same workload's line; per-kernel durations
from a --kernel-trace run; any other counters per kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = ("µs/decode step + effective HBM GB/s, 32 heads, 32K ctx, "
          "2048-token budget")
CSRC = os.path.join(ROOT, "query_aware_kv_amd", "csrc")

# The sources each kernel compiles from: a change to any of them makes the
# recorded HBM traffic of that kernel stale (reported as null).
_ATTN_SRC = ["dev_attn.h", "dev_attn_mfma.h", "common.h", "launch.h"]
KERNELS = {
    "estimate_kernel": ["estimate.hip", "dev_estimate.h", "common.h", "launch.h"],
    "topk_kernel": ["topk.hip", "dev_topk.h", "common.h", "launch.h"],
    "topk_attn_kernel": ["topk_attn.hip", "dev_topk.h"] + _ATTN_SRC,
    "attn_split_kernel": ["attention.hip"] + _ATTN_SRC,
    "attn_merge_kernel": ["attention.hip"] + _ATTN_SRC,
    "union_kernel": ["union.hip", "common.h", "launch.h"],
}
# rocprofv3 counter summaries, one per workload; a line reports the record
# of its own workload only
TRAFFIC_FILES = {
    "longchat": os.path.join(ROOT, "profiles", "hbm_traffic_longchat32k.md"),
    "ragged": os.path.join(ROOT, "profiles", "kernels_ragged_batch.md"),
    "gqa_multistep": os.path.join(ROOT, "profiles", "kernels_gqa_multistep.md"),
}


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


def append_bytes(batch, n_kv_heads, d=128, s=2):
    """One appended token per request: the K and V rows written, and the
    page's min/max read and written back."""
    return batch * n_kv_heads * d * s * (2 + 4)


def attention_recall(torch, q, k_pool, page_table, seq_lens, sel, page_size, sm_scale,
                     top_m=16):
    """How much of full attention a page selection keeps, per (request,
    query head h) of a group of G = Hq / Hkv heads: w = softmax over the
    request's valid tokens t of (q_h . k_t) * sm_scale (float32, outside any
    timed region); `mass` = the sum of w over the tokens of the pages that
    h attends (sel[b][h // G], -1 entries ignored), `top` = the share of the
    top_m highest-weight tokens that lie in those pages.  Returns the mean
    and the minimum of each over every (request, head) with tokens."""
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    S = page_size
    mass, top = [], []
    lens = [int(x) for x in seq_lens.cpu()]
    for b, L in enumerate(lens):
        if L <= 0:
            continue
        n = -(-L // S)
        pages = page_table[b, :n].long()
        keys = k_pool[pages].float()                   # [n, Hkv, S, d]
        keys = keys.permute(1, 0, 2, 3).reshape(Hkv, n * S, d)[:, :L]
        tok_page = torch.arange(L, device=q.device) // S
        m = min(top_m, L)
        for g in range(Hkv):
            kept = torch.zeros(n, dtype=torch.bool, device=q.device)
            js = sel[b, g].long()
            js = js[(js >= 0) & (js < n)]
            kept[js] = True
            kept_tok = kept[tok_page]
            kt = keys[g].t().contiguous()              # [d, L]
            z = torch.matmul(q[b, g * G:(g + 1) * G].float(), kt) * sm_scale
            w = torch.softmax(z, dim=-1)               # [G, L]
            mass += (w * kept_tok).sum(dim=-1).tolist()
            idx = torch.topk(w, m, dim=-1).indices
            top += (kept_tok[idx].float().mean(dim=-1)).tolist()
    return {"mass_mean": sum(mass) / len(mass), "mass_min": min(mass),
            "top%d_mean" % top_m: sum(top) / len(top), "top%d_min" % top_m: min(top)}


def kv_cache_bytes(layers, heads, d, ctx, s=2):
    """K and V of every layer and head for ctx tokens."""
    return layers * 2 * heads * d * ctx * s


def sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, path):
    """(HBM bytes per launch, sources digest) of `kernel` from the committed
    rocprofv3 counter summary at `path`, or (None, digest) if there is none
    or the kernel's sources changed since the counters were taken."""
    digest = sources_digest(KERNELS[kernel])
    try:
        text = open(path).read()
    except OSError:
        return None, digest
    m = re.search(r"^\| %s \| (\d+) \| ([0-9a-f]+) \|" % re.escape(kernel), text, re.M)
    if not m or m.group(2) != digest:
        return None, digest
    return int(m.group(1)), digest


# ------------------------------------------------------------- GPU helpers

def pct(xs, p):
    xs = sorted(xs)
    i = min(len(xs) - 1, max(0, int(round(p / 100 * (len(xs) - 1)))))
    return xs[i]


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def graph_batch(torch, fn, rot, min_steps=100, min_replays=10, warm=2):
    """The timing protocol of every figure in a line: one HIP graph holding
    fn(0), ..., fn(rot - 1) -- one step (or call) on each of the rotating
    caches, back to back -- replayed R >= max(min_replays, min_steps / rot)
    times back to back after `warm` untimed replays.  HIP events on the
    launch stream bracket every replay; the mean is over all R * rot steps,
    the percentiles over the replays' per-step means.  Wall clock (host,
    synchronised on both sides) is reported alongside."""
    g = capture(torch, lambda: [fn(i) for i in range(rot)])
    for _ in range(max(1, warm)):
        g.replay()
    torch.cuda.synchronize()
    R = max(min_replays, -(-min_steps // rot))
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(R):
        g.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e6 / (R * rot)
    per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / rot for i in range(R)]
    mean = ev[0].elapsed_time(ev[R]) * 1e3 / (R * rot)
    del g
    return dict(mean=mean, wall=wall, p10=pct(per, 10), p50=pct(per, 50),
                p90=pct(per, 90), steps=R * rot, replays=R)


def eager_us(torch, fn, rot, n, warm):
    """Wall-clock µs per step of eager issue (the calls from Python through
    ctypes, no graph), synchronised on both sides."""
    for i in range(warm):
        fn(i % rot)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        fn(i % rot)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / n * 1e6


def one_graph_us(torch, fn, rot, n, warm):
    """Wall-clock µs per step of one HIP graph per step, replayed one at a
    time from the host."""
    gs = [capture(torch, lambda i=i: fn(i)) for i in range(rot)]
    for i in range(warm):
        gs[i % rot].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        gs[i % rot].replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / n * 1e6
    del gs
    return us


def stream_read_ceiling(torch, qa, gib=4, reps=10):
    """GB/s of quest_stream_read_probe over a buffer far larger than the
    Infinity Cache."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    qa.quest_stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        qa.quest_stream_read_probe(buf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    gbps = (gib << 30) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbps, 1)


def make_layer(qa, synth, wl, layer=0, dev="cuda"):
    c = synth.draw_layer(wl, layer, dev)
    kv = qa.paged_kv(wl.batch, wl.num_q_heads, wl.num_kv_heads,
                     wl.pool_pages(), wl.max_pages, wl.torch_dtype,
                     page_size=wl.page_size)
    kmin, kmax = qa.alloc_meta(kv)
    qa.quest_update_page_meta(kv, c["k_pool"], c["v_pool"], kmin, kmax,
                              c["page_table"], c["seq_lens"])
    c.update(kmin=kmin, kmax=kmax, kv=kv)
    return c


def time_single_layer(args, torch, qa, synth, wls, with_dense=True, full=True):
    """Sparse step (and dense baseline) over rotating instances of one layer
    geometry, every figure by the back-to-back graph protocol
    (graph_batch); each kernel of the step timed alone the same way;
    algorithmic bytes from the selections actually made."""
    rot = len(wls)
    insts = [make_layer(qa, synth, wl) for wl in wls]
    torch.cuda.synchronize()
    kv = insts[0]["kv"]
    k = wls[0].k_pages
    sm = 1.0 / math.sqrt(128)
    steps = [qa.SparseDecodeStep(kv, k, sm, select=args.select) for _ in range(rot)]
    denses = [qa.DenseDecode(kv, sm) for _ in range(rot)] if with_dense else []
    min_steps = max(100, args.steps)
    warm = max(1, -(-args.warmup // rot))

    def step_call(i, sts=steps):
        c = insts[i]
        sts[i](c["q"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"],
               c["page_table"], c["seq_lens"])

    def dense_call(i):
        c = insts[i]
        denses[i](c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])

    for i in range(rot):                 # eager warm-up before capture
        step_call(i)
        if with_dense:
            dense_call(i)
    torch.cuda.synchronize()
    t_batch = graph_batch(torch, step_call, rot, min_steps, warm=warm)
    t_eager = t_graph1 = None
    if full:                             # other ways of issuing, not the value
        t_eager = eager_us(torch, step_call, rot, min(args.steps, 200), args.warmup)
        t_graph1 = one_graph_us(torch, step_call, rot, min(args.steps, 200),
                                args.warmup)
    by_select = {steps[0].select: round(t_batch["mean"], 3)}
    if full:
        for mode in ("attention", "separate"):
            if mode in by_select:
                continue
            alt = [qa.SparseDecodeStep(kv, k, sm, select=mode) for _ in range(rot)]
            for i in range(rot):
                step_call(i, alt)
            torch.cuda.synchronize()
            by_select[mode] = round(graph_batch(torch, lambda i: step_call(i, alt),
                                                rot, min_steps, warm=1)["mean"], 3)
            del alt
    t_dense = None
    if with_dense:
        t_dense = graph_batch(torch, dense_call, rot, min_steps=2 * rot,
                              min_replays=3, warm=1)

    def est(i):
        c, st = insts[i], steps[i]
        qa.quest_estimate(kv, c["q"], c["kmin"], c["kmax"], c["page_table"],
                          c["seq_lens"], st.scores)

    def ta_splits(i):
        c, st = insts[i], steps[i]
        qa.quest_topk_sparse_decode_attn_splits(
            kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"],
            st.scores, k, 0, 0, sm, st.sel, st.out, st.workspace)

    def merge(i):
        st = steps[i]
        qa.quest_merge_attn_splits(kv, k, st.workspace, st.out)

    def topk_attn(i):
        c, st = insts[i], steps[i]
        qa.quest_topk_sparse_decode_attn(
            kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"],
            c["seq_lens"], st.scores, k, sm, st.sel, st.out, st.workspace)

    def topk_attn_forced(i):   # the pages' default: 2 sink + 2 local pages
        c, st = insts[i], steps[i]
        qa.quest_topk_sparse_decode_attn_ex(
            kv, c["q"], c["k_pool"], c["v_pool"], c["page_table"],
            c["seq_lens"], st.scores, k, 2, 2, sm, st.sel, st.out, st.workspace)

    def topk_sep(i):
        c, st = insts[i], steps[i]
        qa.quest_topk_pages(kv, st.scores, c["seq_lens"], k, st.sel)

    def attn_sep(i):
        c, st = insts[i], steps[i]
        qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                    c["page_table"], c["seq_lens"], st.sel, k,
                                    sm, st.out, st.workspace)

    mode = steps[0].select
    fits = kv.max_pages_per_seq <= qa.TOPK_ATTN_MAX_PAGES
    ku = {}                              # per-kernel (per-call) device µs
    ku["estimate_kernel"] = graph_batch(torch, est, rot, min_steps, warm=1)["mean"]
    if mode == "attention":
        ku["topk_attn_kernel"] = graph_batch(torch, ta_splits, rot, min_steps,
                                             warm=1)["mean"]
        ku["attn_merge_kernel"] = graph_batch(torch, merge, rot, min_steps,
                                              warm=1)["mean"]
    else:
        ku["topk_kernel"] = graph_batch(torch, topk_sep, rot, min_steps, warm=1)["mean"]
        # attn_split_kernel and its merge: one call, timed together
        ku["attn_split_kernel+attn_merge_kernel"] = graph_batch(
            torch, attn_sep, rot, min_steps, warm=1)["mean"]
    other = {}
    if full:
        if mode == "attention":
            other["quest_topk_pages"] = graph_batch(torch, topk_sep, rot, min_steps,
                                                    warm=1)["mean"]
            other["quest_sparse_decode_attn"] = graph_batch(torch, attn_sep, rot,
                                                            min_steps, warm=1)["mean"]
        if fits:
            other["quest_topk_sparse_decode_attn"] = graph_batch(
                torch, topk_attn, rot, min_steps, warm=1)["mean"]
            other["quest_topk_sparse_decode_attn_ex (2 sink + 2 local pages)"] = \
                graph_batch(torch, topk_attn_forced, rot, min_steps, warm=1)["mean"]
    for i in range(rot):                 # leave the plain selection in every step
        topk_sep(i)
    torch.cuda.synchronize()

    sels = [st.sel.cpu().numpy() for st in steps]
    lens_all = [[int(x) for x in c["seq_lens"].cpu()] for c in insts]
    bstep = [step_bytes(lens_all[i], kv.num_kv_heads, kv.num_q_heads, k, sel=sels[i],
                        page_size=kv.page_size)
             for i in range(rot)]
    avg = {key: sum(b[key] for b in bstep) / rot for key in bstep[0]}
    kb = kernel_bytes(avg, kv, k)
    dbytes = sum(dense_bytes(l, kv.num_kv_heads, kv.num_q_heads, page_size=kv.page_size)
                 for l in lens_all) / rot
    return dict(t_batch=t_batch, t_eager=t_eager, t_graph1=t_graph1, t_dense=t_dense,
                bytes=avg, kernel_us=ku, kernel_bytes=kb, other_us=other,
                by_select=by_select, dense_bytes=dbytes, insts=insts, kv=kv,
                k_pages=k, sm=sm, mode=mode)


def topk_attn_splits(rows, k):
    """Workgroups per row of the Top-K + attention launch (its plan: 8 waves,
    2 pages per wave if that still gives >= 256 workgroups, else 1)."""
    ppw = 2 if rows * -(-k // 16) >= 256 else 1
    return max(1, -(-k // (8 * ppw)))


def kernel_bytes(avg, kv, k):
    """Per kernel of the step, per launch: (algorithmic bytes, overhead
    bytes).  Algorithmic bytes follow the step's byte model -- each page's
    metadata, the kept pages' valid K/V, q, the output and the page-table
    entries -- split over the kernels that must move them; the score and
    selection round trips and the split partials are implementation
    overhead, reported apart and not counted."""
    B, Hq, Hkv = kv.batch, kv.num_q_heads, kv.num_kv_heads
    scores = B * Hkv * kv.max_pages_per_seq * 4
    sel = B * Hkv * k * 4
    partials = B * Hq * topk_attn_splits(B * Hkv, k) * (128 + 2) * 4
    return {
        "estimate_kernel": (avg["meta"] + avg["q"] + avg["table"],
                            {"scores_written": scores}),
        "topk_attn_kernel": (avg["kv"] + avg["q"],
                             {"scores_read": scores, "sel_written": sel,
                              "kept_table_entries": sel, "partials_written": partials}),
        "attn_merge_kernel": (avg["out"], {"partials_read": partials}),
        "topk_kernel": (0, {"scores_read": scores, "sel_written": sel}),
        "attn_split_kernel+attn_merge_kernel": (
            avg["kv"] + avg["q"] + avg["out"],
            {"sel_read": sel, "kept_table_entries": sel, "partials": 2 * partials}),
    }


def roofline(ku, kb, traffic_file=None):
    """Roofline of the kernel with the most time per step: algorithmic bytes
    per launch (the step's byte model, kernel_bytes) over its HIP-event
    time, against the 8 TB/s HBM peak.  `traffic` is the rocprofv3 counter
    figure that `traffic_file` (the same workload's summary in profiles/)
    records for that kernel while its sources are unchanged, else null; it
    is not measured in this run."""
    dom = max(ku, key=lambda n: ku[n])
    us = ku[dom]
    alg, over = kb[dom]
    achieved = alg / (us * 1e-6) / 1e9
    # a call of several kernels ("a+b"): the sum of their records
    parts = [p_.strip() for p_ in dom.split("+")]
    traffic, digest = None, None
    if traffic_file and all(p_ in KERNELS for p_ in parts):
        recs = [recorded_traffic(p_, traffic_file) for p_ in parts]
        digest = ",".join(r_[1] for r_ in recs)
        if all(r_[0] is not None for r_ in recs):
            traffic = sum(r_[0] for r_ in recs)
    return {"bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": (f"recorded: {os.path.relpath(traffic_file, ROOT)} "
                               f"(rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated), "
                               f"sources digest {digest}" if traffic is not None else
                               "null: no counter record of this workload for the "
                               "current sources"),
            "kernel": dom, "kernel_us": round(us, 3),
            "bytes_per_launch": int(alg),
            "overhead_bytes_per_launch": {k_: int(v) for k_, v in over.items()}}


def protocol_note(r, rot):
    tb = r["t_batch"]
    return (f"value = mean µs per step over {tb['steps']} steps: {tb['replays']} "
            f"back-to-back replays of one HIP graph holding one step on each of "
            f"{rot} rotating caches (HIP events on the launch stream around every "
            f"replay, untimed warm-up replays first); p10/p50/p90 over the "
            f"replays' per-step means; every kernel and the dense baseline timed "
            f"the same way; eager issue and one-graph-per-step are reported apart "
            f"and are not the value")


# ------------------------------------------------------------- workloads

def bench_longchat(args, torch, qa, synth):
    base = synth.longchat_layer_workload()
    wls = [synth.longchat_layer_workload(seed=base.base_seed + 1000 * i)
           for i in range(args.rotate)]
    r = time_single_layer(args, torch, qa, synth, wls, with_dense=not args.no_dense)
    tb = r["t_batch"]
    us = tb["mean"]
    gbps = r["bytes"]["total"] / (us * 1e-6) / 1e9
    us_dense = r["t_dense"]["mean"] if r["t_dense"] else float("nan")
    ceiling = None if args.no_ceiling else stream_read_ceiling(torch, qa)
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
        "timed_steps": tb["steps"],
        "step_us_p10_p50_p90": [round(tb[p], 3) for p in ("p10", "p50", "p90")],
        "wall_us_per_step": round(tb["wall"], 3),
        "effective_GBps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "stream_read_GBps": ceiling,
        "ceiling_frac": round(gbps / ceiling, 4) if ceiling else None,
        "bytes_per_step": int(r["bytes"]["total"]),
        "dense_us_per_step": round(us_dense, 3),
        "speedup_vs_dense": round(us_dense / us, 3),
        "dense_effective_GBps": round(r["dense_bytes"] / (us_dense * 1e-6) / 1e9, 1),
        "timing": protocol_note(r, args.rotate),
        "eager_us_per_step": round(r["t_eager"], 3),
        "one_graph_per_step_us": round(r["t_graph1"], 3),
        "step_us_by_select": r["by_select"],
        "kernel_us": {n: round(v, 3) for n, v in r["kernel_us"].items()},
        "other_call_us": {n: round(v, 3) for n, v in r["other_us"].items()},
        "roofline": roofline(r["kernel_us"], r["kernel_bytes"], TRAFFIC_FILES["longchat"]),
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(r, args.cpu_seconds)
        if not args.no_cpu_all_cores:
            line["cpu_baseline"]["all_cores"] = cpu_baseline_all_cores(r, args.cpu_seconds)
    del r
    torch.cuda.empty_cache()
    if not args.no_extra:
        line["extra"] = extra_workloads(args, torch, qa, synth)
    return line


def single_layer_line(r, rot, traffic_file=None):
    """The figures every single-layer workload reports."""
    tb = r["t_batch"]
    us = tb["mean"]
    us_dense = r["t_dense"]["mean"] if r["t_dense"] else None
    d = {"us_per_step": round(us, 3),
         "step_us_p10_p50_p90": [round(tb[p], 3) for p in ("p10", "p50", "p90")],
         "timed_steps": tb["steps"], "rotating_caches": rot,
         "bytes_per_step": int(r["bytes"]["total"]),
         "effective_GBps": round(r["bytes"]["total"] / (us * 1e-6) / 1e9, 1),
         "hbm_frac": round(r["bytes"]["total"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
         "kernel_us": {n: round(v, 3) for n, v in r["kernel_us"].items()},
         "roofline": roofline(r["kernel_us"], r["kernel_bytes"], traffic_file)}
    if us_dense:
        d.update(dense_us_per_step=round(us_dense, 3),
                 speedup_vs_dense=round(us_dense / us, 3),
                 dense_effective_GBps=round(r["dense_bytes"] / (us_dense * 1e-6) / 1e9, 1))
    return d


def bench_ragged(args, torch, qa, synth, full=True):
    wl = synth.ragged_batch_workload()
    r = time_single_layer(args, torch, qa, synth, [wl],
                          with_dense=not args.no_dense and full, full=full)
    d = single_layer_line(r, 1, TRAFFIC_FILES["ragged"])
    d["config"] = {"workload": "ragged_batch_decode", "batch": wl.batch,
                   "q_heads": 32, "kv_heads": 32, "ctx_min": min(wl.seq_lens),
                   "ctx_max": max(wl.seq_lens), "budget_tokens": 2048,
                   "dtype": "bf16", "select": r["mode"]}
    if not full:
        return d
    us = d["us_per_step"]
    line = {
        "metric": "µs/decode step + effective HBM GB/s, batched ragged",
        "value": us, "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q; pool pages permuted)",
        "config": d.pop("config"),
        "timing": protocol_note(r, 1) + " (one cache: its 1.6 GiB of touched "
                  "bytes far exceed the Infinity Cache)",
        "eager_us_per_step": round(r["t_eager"], 3),
        "one_graph_per_step_us": round(r["t_graph1"], 3),
        "step_us_by_select": r["by_select"],
        "other_call_us": {n: round(v, 3) for n, v in r["other_us"].items()},
        "gpu": torch.cuda.get_device_name(0)}
    line.update(d)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_ragged(r, args.cpu_seconds)
    return line


def sweep_point(args, torch, qa, synth, ctx, budget, full=True):
    # enough independent caches that the bytes one pass over them touches
    # (metadata + selected pages) exceed the Infinity Cache
    touched_mib = ctx / 1024 + min(budget, ctx) / 64
    rot = min(64, max(2, math.ceil(768 / touched_mib)))
    wls = [synth.sweep_workload(ctx, budget, seed=2 + 1000 * i) for i in range(rot)]
    r = time_single_layer(args, torch, qa, synth, wls,
                          with_dense=not args.no_dense, full=False)
    d = single_layer_line(r, rot)
    d.update(ctx=ctx, budget=budget)
    del r
    torch.cuda.empty_cache()
    return d


def bench_sweep(args, torch, qa, synth):
    points = []
    for ctx in synth.SWEEP_CTX:
        for budget in synth.SWEEP_BUDGET:
            points.append(sweep_point(args, torch, qa, synth, ctx, budget))
            print(json.dumps({"progress": points[-1]}), file=sys.stderr, flush=True)
    at = [p for p in points if p["ctx"] == 32768 and p["budget"] == 2048][0]
    return {
        "metric": "µs/decode step over context x budget, 32 heads",
        "value": at["us_per_step"], "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(at["us_per_step"] / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (as longchat, per point)",
        "config": {"workload": "ctx_budget_sweep", "ctx": list(synth.SWEEP_CTX),
                   "budget_tokens": list(synth.SWEEP_BUDGET),
                   "value_at": "ctx 32768, budget 2048"},
        "timing": "each point as the headline: back-to-back replays of one HIP "
                  "graph over its rotating caches, >= 100 steps",
        "roofline": at["roofline"],
        "points": points, "gpu": torch.cuda.get_device_name(0)}


def bench_gqa_multistep(args, torch, qa, synth, full=True):
    wl = synth.gqa_multistep_workload()
    dev = "cuda"
    sm = 1.0 / math.sqrt(128)
    k = wl.k_pages
    nsteps = wl.steps
    layers = []
    for layer in range(wl.layers):
        c = make_layer(qa, synth, wl, layer)
        st = dict(c=c, kv=c["kv"])
        if layer < wl.dense_layers:
            st["dense"] = qa.DenseDecode(c["kv"], sm)
        else:
            st["step"] = qa.SparseDecodeStep(c["kv"], k, sm, select=args.select)
        st["q"] = torch.stack([synth.draw_query(wl, layer, dev, step=s)
                               for s in range(nsteps)])
        kn, vn = zip(*[synth.draw_append_token(wl, layer, s, dev)
                       for s in range(nsteps)])
        st["k_new"], st["v_new"] = torch.stack(kn), torch.stack(vn)
        layers.append(st)
    L0 = wl.seq_lens[0]
    lens = [torch.tensor([L0 + s + 1], dtype=torch.int32, device=dev)
            for s in range(nsteps)]
    torch.cuda.synchronize()

    def one_step(s):
        for layer, st in enumerate(layers):
            c, kv = st["c"], st["kv"]
            if layer < wl.dense_layers:   # the append rides on the attention launch
                st["dense"].append_step(st["q"][s], c["k_pool"], c["v_pool"],
                                        c["kmin"], c["kmax"], c["page_table"],
                                        lens[s], st["k_new"][s], st["v_new"][s])
            else:   # the append rides on the estimate launch
                st["step"].append_step(st["q"][s], c["k_pool"], c["v_pool"],
                                       c["kmin"], c["kmax"], c["page_table"],
                                       lens[s], st["k_new"][s], st["v_new"][s])

    # Warm-up steps re-append the same tokens at the same positions; they
    # leave every page box a superset of the timed run's, which changes no
    # byte count and no launch.
    for s in range(min(args.warmup, nsteps)):
        one_step(s)
    torch.cuda.synchronize()
    us_eager = None
    if full:
        t0 = time.perf_counter()
        for s in range(nsteps):
            one_step(s)
        torch.cuda.synchronize()
        us_eager = (time.perf_counter() - t0) / nsteps * 1e6
    # the protocol: one graph per 32-layer step (128 of them, each appending
    # its own token), replayed back to back in step order, events around each
    graphs = [capture(torch, lambda s=s: one_step(s)) for s in range(nsteps)]
    for s in range(min(args.warmup, nsteps)):
        graphs[s].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
    ev[0].record(stream)
    for s in range(nsteps):
        graphs[s].replay()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[s].elapsed_time(ev[s + 1]) * 1e3 for s in range(nsteps)]
    us = ev[0].elapsed_time(ev[nsteps]) * 1e3 / nsteps
    del graphs

    # bytes per step (final lengths, selections of the last replayed step)
    B = 1
    sparse_b = 0
    for st in layers[wl.dense_layers:]:
        sel = st["step"].sel.cpu().numpy()
        sparse_b += step_bytes([L0 + nsteps], 8, 32, k, sel=sel)["total"]
    dense_b = wl.dense_layers * dense_bytes([L0 + nsteps], 8, 32)
    app_b = wl.layers * append_bytes(B, 8)
    total = sparse_b + dense_b + app_b
    all_dense = wl.layers * dense_bytes([L0 + nsteps], 8, 32) + app_b

    # the layers' kernels at the last step, one by one: a graph of one call
    # per layer over every sparse (or dense) layer, back to back, so that
    # each reads its bytes from HBM (30 sparse layers: 0.5 GB); the roofline
    # is that of the kernel with the most time per 32-layer step
    s_l = nsteps - 1
    sparse_l = layers[wl.dense_layers:]
    dense_l = layers[:wl.dense_layers]
    Lf = L0 + nsteps

    def ae(i):
        sp = sparse_l[i]
        c, st = sp["c"], sp["step"]
        qa.quest_append_estimate(sp["kv"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"],
                                 c["page_table"], lens[s_l], sp["k_new"][s_l],
                                 sp["v_new"][s_l], sp["q"][s_l], st.scores)

    def ta(i):
        sp = sparse_l[i]
        c, st = sp["c"], sp["step"]
        qa.quest_topk_sparse_decode_attn_splits(
            sp["kv"], sp["q"][s_l], c["k_pool"], c["v_pool"], c["page_table"],
            lens[s_l], st.scores, k, 0, 0, sm, st.sel, st.out, st.workspace)

    def mg(i):
        sp = sparse_l[i]
        qa.quest_merge_attn_splits(sp["kv"], k, sp["step"].workspace, sp["step"].out)

    def da(i):
        de = dense_l[i]
        c, d_ = de["c"], de["dense"]
        qa.quest_append_decode_attn(de["kv"], c["k_pool"], c["v_pool"], c["kmin"],
                                    c["kmax"], c["page_table"], lens[s_l],
                                    de["k_new"][s_l], de["v_new"][s_l], de["q"][s_l],
                                    sm, d_.out, d_.workspace)

    ns = len(sparse_l)
    ku = {"estimate_kernel (append)": graph_batch(torch, ae, ns, 100, warm=1)["mean"],
          "topk_attn_kernel": graph_batch(torch, ta, ns, 100, warm=1)["mean"],
          "attn_merge_kernel": graph_batch(torch, mg, ns, 100, warm=1)["mean"],
          "attn_split_kernel+attn_merge_kernel (dense)":
              graph_batch(torch, da, len(dense_l), 20, min_replays=5, warm=1)["mean"]}
    sb = step_bytes([Lf], 8, 32, k, sel=sparse_l[0]["step"].sel.cpu().numpy())
    mp = sparse_l[0]["kv"].max_pages_per_seq
    kb = kernel_bytes(sb, sparse_l[0]["kv"], k)
    kb["estimate_kernel (append)"] = (sb["meta"] + sb["q"] + sb["table"] + append_bytes(1, 8),
                                      {"scores_written": 8 * mp * 4})
    kb["attn_split_kernel+attn_merge_kernel (dense)"] = (dense_bytes([Lf], 8, 32)
                                                         + append_bytes(1, 8), {})
    per_step = {"estimate_kernel (append)": wl.layers - wl.dense_layers,
                "topk_attn_kernel": wl.layers - wl.dense_layers,
                "attn_merge_kernel": wl.layers - wl.dense_layers,
                "attn_split_kernel+attn_merge_kernel (dense)": wl.dense_layers}
    dom = max(ku, key=lambda c_: ku[c_] * per_step[c_])
    rl = roofline({dom: ku[dom]}, {dom: kb[dom]}, TRAFFIC_FILES["gqa_multistep"])
    d = {"us_per_step": round(us, 3),
         "step_us_p10_p50_p90": [round(pct(per, q_), 3) for q_ in (10, 50, 90)],
         "timed_steps": nsteps,
         "bytes_per_step": int(total),
         "effective_GBps": round(total / (us * 1e-6) / 1e9, 1),
         "hbm_frac": round(total / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
         "all_dense_bytes_per_step": int(all_dense),
         "launches_per_step": wl.dense_layers * 2 + (wl.layers - wl.dense_layers) * 3,
         "layer_kernel_us": {c_: round(v, 3) for c_, v in ku.items()},
         "roofline": rl,
         "config": {"workload": "gqa_multistep_decode", "layers": wl.layers,
                    "q_heads": 32, "kv_heads": 8, "ctx_start": L0,
                    "appended_steps": nsteps, "budget_tokens": wl.budget_tokens,
                    "dense_layers": wl.dense_layers}}
    if not full:
        return d
    line = {
        "metric": "µs per 32-layer decode step, GQA 32/8, 32K ctx, "
                  "2048-token budget, layers 0-1 dense",
        "value": d["us_per_step"], "unit": "us/step", "n_gpus": 1,
        "steps": nsteps, "warmup": min(args.warmup, nsteps),
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) fp16, 4 outlier channels x8 per "
                "(layer, kv-head); one appended token per layer per step)",
        "timing": "value = mean µs per 32-layer step over the 128 appended "
                  "steps: one HIP graph per step, replayed back to back in step "
                  "order, HIP events around each replay; eager issue reported "
                  "apart",
        "eager_us_per_step": round(us_eager, 3),
        "gpu": torch.cuda.get_device_name(0),
    }
    line.update(d)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_multistep(layers, wl, args.cpu_seconds)
    return line


def bench_gqa_union(args, torch, qa, synth):
    """One GQA layer (32 q-heads / 8 kv-heads, 32K, 2048-token budget): the
    group-sum rule against the per-head + union rule, same caches: time,
    bytes, and how much of full attention each rule's pages hold
    (attention_recall)."""
    rot = args.rotate
    wls = [synth.gqa_multistep_workload(seed=4 + 1000 * i, layers=1, steps=0)
           for i in range(rot)]
    insts = [make_layer(qa, synth, wl) for wl in wls]
    torch.cuda.synchronize()
    kv = insts[0]["kv"]
    k = wls[0].k_pages
    sm = 1.0 / math.sqrt(128)
    G = kv.num_q_heads // kv.num_kv_heads
    sums = [qa.SparseDecodeStep(kv, k, sm) for _ in range(rot)]
    unions = [qa.UnionDecodeStep(kv, k, sm) for _ in range(rot)]   # fused union
    seps = [qa.UnionDecodeStep(kv, k, sm, fused=False) for _ in range(rot)]

    def call(steps, i):
        c = insts[i]
        steps[i](c["q"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"],
                 c["page_table"], c["seq_lens"])

    res = {}
    for name, steps in (("sum", sums), ("union", unions), ("union_separate", seps)):
        for i in range(rot):
            call(steps, i)
        torch.cuda.synchronize()
        t = graph_batch(torch, lambda i, steps=steps: call(steps, i), rot,
                        max(100, args.steps), warm=1)
        lens = [int(x) for x in insts[0]["seq_lens"].cpu()]
        b = [step_bytes(lens, kv.num_kv_heads, kv.num_q_heads, k,
                        sel=steps[i].sel.cpu().numpy())["total"] for i in range(rot)]
        kept = [float((steps[i].sel >= 0).sum()) / (kv.batch * kv.num_kv_heads)
                for i in range(rot)]
        res[name] = dict(us=t["mean"], bytes=sum(b) / rot,
                         pages=sum(kept) / rot)
    u, sm_, us = res["union"], res["sum"], res["union_separate"]

    # the union step's calls one by one, for its roofline
    def e_heads(i):
        c, st = insts[i], unions[i]
        qa.quest_estimate_heads(kv, c["q"], c["kmin"], c["kmax"], c["page_table"],
                                c["seq_lens"], st.scores)

    def tk_heads(i):
        c, st = insts[i], unions[i]
        qa.quest_topk_pages_ex(st.kv_heads, st.scores, c["seq_lens"], k, 0, 0,
                               st.sel_heads)

    def un(i):
        st = unions[i]
        qa.quest_union_pages(kv, st.sel_heads, k, st.sel)

    def att(i):
        c, st = insts[i], unions[i]
        qa.quest_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                    c["page_table"], c["seq_lens"], st.sel, G * k,
                                    sm, st.out, st.workspace)

    def un_att(i):
        c, st = insts[i], unions[i]
        qa.quest_union_sparse_decode_attn(kv, c["q"], c["k_pool"], c["v_pool"],
                                          c["page_table"], c["seq_lens"], st.sel_heads,
                                          k, sm, st.sel, st.out, st.workspace)

    t_calls = {name: graph_batch(torch, f, rot, 100, warm=1)["mean"] for name, f in (
        ("quest_estimate_heads", e_heads), ("quest_topk_pages", tk_heads),
        ("quest_union_pages", un), ("quest_sparse_decode_attn", att),
        ("quest_union_sparse_decode_attn", un_att))}
    lens = [int(x) for x in insts[0]["seq_lens"].cpu()]
    Hq, Hkv, mp = kv.num_q_heads, kv.num_kv_heads, kv.max_pages_per_seq
    sb = step_bytes(lens, Hkv, Hq, k, sel=unions[0].sel.cpu().numpy())
    # per call (one kernel each, but the attention call: split + merge)
    names = {"quest_estimate_heads": "estimate_kernel (per head)",
             "quest_topk_pages": "topk_kernel",
             "quest_union_pages": "union_kernel",
             "quest_sparse_decode_attn": "attn_split_kernel+attn_merge_kernel",
             "quest_union_sparse_decode_attn":
                 "attn_split_kernel+attn_merge_kernel (union inside)"}
    b_calls = {
        "quest_estimate_heads": (sb["meta"] + sb["q"] + sb["table"],
                                 {"scores_written": Hq * mp * 4}),
        "quest_topk_pages": (0, {"scores_read": Hq * mp * 4, "sel_written": Hq * k * 4}),
        "quest_union_pages": (0, {"sel_read": Hq * k * 4, "union_written": Hkv * G * k * 4}),
        "quest_sparse_decode_attn": (sb["kv"] + sb["q"] + sb["out"],
                                     {"sel_read": Hkv * G * k * 4}),
        "quest_union_sparse_decode_attn": (sb["kv"] + sb["q"] + sb["out"],
                                           {"sel_heads_read": Hq * k * 4,
                                            "union_written": Hkv * G * k * 4})}
    # the roofline: the step's calls but the two the fused call replaces
    step_calls = [c_ for c_ in t_calls
                  if c_ not in ("quest_union_pages", "quest_sparse_decode_attn")]
    ku = {names[c_]: t_calls[c_] for c_ in step_calls}
    kb = {names[c_]: b_calls[c_] for c_ in step_calls}
    # what each rule keeps of full attention, on every rotating cache
    rec = {}
    for name, steps in (("group_sum", sums), ("union", unions)):
        per = [attention_recall(torch, insts[i]["q"], insts[i]["k_pool"],
                                insts[i]["page_table"], insts[i]["seq_lens"],
                                steps[i].sel, kv.page_size, sm) for i in range(rot)]
        rec[name] = {}
        for m_ in per[0]:
            vals = [r[m_] for r in per]
            rec[name][m_] = round(sum(vals) / len(vals) if m_.endswith("mean")
                                  else min(vals), 4)
    return {
        "metric": "µs/decode step, GQA 32/8 layer, per-head Top-K + union vs "
                  "group-sum Top-K",
        "value": round(u["us"], 3), "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(u["us"] / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded N(0,1) fp16, 4 outlier channels x8 per kv-head)",
        "config": {"workload": "gqa_layer_union_rule", "batch": 1, "q_heads": 32,
                   "kv_heads": 8, "ctx": 32768, "budget_tokens": 2048,
                   "rotating_caches": rot},
        "union": {"us_per_step": round(u["us"], 3), "bytes_per_step": int(u["bytes"]),
                  "effective_GBps": round(u["bytes"] / (u["us"] * 1e-6) / 1e9, 1),
                  "pages_per_kv_head": round(u["pages"], 1),
                  "step": "quest_estimate_heads, quest_topk_pages_ex per query head, "
                          "quest_union_sparse_decode_attn (the union built inside "
                          "the attention launch)"},
        "union_separate_us_per_step": round(us["us"], 3),
        "group_sum": {"us_per_step": round(sm_["us"], 3),
                      "bytes_per_step": int(sm_["bytes"]),
                      "effective_GBps": round(sm_["bytes"] / (sm_["us"] * 1e-6) / 1e9, 1),
                      "pages_per_kv_head": round(sm_["pages"], 1)},
        "union_pages_over_k": round(u["pages"] / k, 3),
        "attention_recall": dict(rec, note="per (request, query head): the full-attention "
                                 "weight (float32 softmax over every valid token) on the "
                                 "pages the head attends, and the share of its 16 "
                                 "highest-weight tokens in them; mean and min over heads "
                                 "and rotating caches; synthetic data"),
        "union_call_us": {c_: round(v, 3) for c_, v in t_calls.items()},
        "roofline": roofline(ku, kb),
        "group": G, "gpu": torch.cuda.get_device_name(0)}


def bench_page32(args, torch, qa, synth):
    """Page size 16 against 32 ("Guide to Quest", Best Practices 1) on the
    LongChat layer at 32K and 128K with the same 2048-token budget, and the
    one-shot prefill metadata build against writing the prompt's K."""
    import dataclasses
    rows = []
    for ctx in (32768, 131072):
        for S in (16, 32):
            touched_mib = ctx / 1024 * 16 / S + 2048 / 64
            rot = min(args.rotate, max(2, math.ceil(768 / touched_mib)))
            wls = [dataclasses.replace(synth.longchat_layer_workload(ctx, 2048,
                                                                     seed=1 + 1000 * i),
                                       page_size=S, name=f"p{S}_ctx{ctx}")
                   for i in range(rot)]
            r = time_single_layer(args, torch, qa, synth, wls,
                                  with_dense=not args.no_dense, full=False)
            us = r["t_batch"]["mean"]
            c, kv = r["insts"][0], r["kv"]
            # prefill: rebuild every box of the prompt vs writing its K once
            kmin, kmax = qa.alloc_meta(kv)
            k_bytes = c["k_pool"].numel() * c["k_pool"].element_size()
            dst = torch.empty_like(c["k_pool"])
            stream = torch.cuda.current_stream()

            def ev(fn, reps=10):
                fn()
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) * 1e3 / reps

            meta_us = ev(lambda: qa.quest_update_page_meta(
                kv, c["k_pool"], c["v_pool"], kmin, kmax, c["page_table"],
                c["seq_lens"]))
            kwrite_us = ev(lambda: dst.fill_(1.0))
            meta_bytes = k_bytes + 2 * kv.num_pool_pages * kv.num_kv_heads * 128 * 2
            rows.append({
                "ctx": ctx, "page_size": S, "k_pages": wls[0].k_pages,
                "us_per_step": round(us, 3),
                "bytes_per_step": int(r["bytes"]["total"]),
                "effective_GBps": round(r["bytes"]["total"] / (us * 1e-6) / 1e9, 1),
                "meta_bytes_per_step": int(r["bytes"]["meta"]),
                "dense_us": round(r["t_dense"]["mean"], 3) if r["t_dense"] else None,
                "kernel_us": {k_: round(v, 3) for k_, v in r["kernel_us"].items()},
                "roofline": roofline(r["kernel_us"], r["kernel_bytes"]),
                "prefill_meta_build_us": round(meta_us, 2),
                "prefill_meta_GBps": round(meta_bytes / (meta_us * 1e-6) / 1e9, 1),
                "prefill_k_write_us": round(kwrite_us, 2),
                "meta_build_over_k_write": round(meta_us / kwrite_us, 3)})
            print(json.dumps({"progress": rows[-1]}), file=sys.stderr, flush=True)
            del r, c, dst, kmin, kmax
            torch.cuda.empty_cache()
    at = [x for x in rows if x["ctx"] == 131072 and x["page_size"] == 32][0]
    return {
        "metric": "µs/decode step with 32-token pages, 32 heads, 128K ctx, "
                  "2048-token budget (16-token pages alongside)",
        "value": at["us_per_step"], "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(at["us_per_step"] / 1e3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic (as longchat, per point)",
        "config": {"workload": "page_size_16_vs_32", "ctx": [32768, 131072],
                   "page_size": [16, 32], "budget_tokens": 2048,
                   "value_at": "ctx 131072, page size 32"},
        "roofline": at["roofline"],
        "points": rows, "gpu": torch.cuda.get_device_name(0)}


def bench_head_groups(args, torch, qa, synth):
    """The LongChat layer split into 1, 2 or 4 head groups, each group an
    estimate -> Top-K + attention chain over its own caches (32 / groups
    heads each, so the bytes per step equal the headline's).  The chains run
    one after another on one stream ("serial") or as parallel branches of
    one HIP graph, one default-priority stream per group ("parallel"): does
    overlapping one group's selection and K/V stream with another group's
    bounds pay?  Same protocol as the headline (back-to-back graph replays
    over rotating caches, >= --steps steps)."""
    import dataclasses
    rot = 8
    variants = args.hg_variants.split(",")
    side = [torch.cuda.Stream() for _ in range(4)]   # default priority
    sm = 1.0 / math.sqrt(128)
    out = {}
    for ng in (1, 2, 4):
        hk = 32 // ng
        caches = []
        for r in range(rot):
            grp = []
            for gi in range(ng):
                wl = dataclasses.replace(synth.longchat_layer_workload(seed=1 + 1000 * r + 97 * gi),
                                         num_q_heads=hk, num_kv_heads=hk,
                                         name=f"head_groups{ng}_{r}_{gi}")
                c = make_layer(qa, synth, wl)
                grp.append((c, qa.SparseDecodeStep(c["kv"], wl.k_pages, sm, select="attention")))
            caches.append(grp)

        def chain(c, st):
            st(c["q"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"], c["page_table"],
               c["seq_lens"])

        def serial(i):
            for c, st in caches[i]:
                chain(c, st)

        def parallel(i):
            main = torch.cuda.current_stream()
            for j, (c, st) in enumerate(caches[i]):
                side[j].wait_stream(main)
                with torch.cuda.stream(side[j]):
                    chain(c, st)
            for j in range(len(caches[i])):
                main.wait_stream(side[j])

        for i in range(rot):
            serial(i)
        torch.cuda.synchronize()
        for v, fn in (("serial", serial), ("parallel", parallel)):
            if v not in variants or (v == "parallel" and ng == 1):
                continue
            t = graph_batch(torch, fn, rot, max(args.steps, 100))
            out[f"{v}_{ng}_groups"] = {
                "us_per_step": round(t["mean"], 3),
                "step_us_p10_p50_p90": [round(t[p_], 3) for p_ in ("p10", "p50", "p90")],
                "timed_steps": t["steps"]}
            print(json.dumps({"progress": f"{v}_{ng}_groups", "us_per_step": t["mean"]}),
                  file=sys.stderr, flush=True)
        del caches
        torch.cuda.empty_cache()
    one = out.get("serial_1_groups", {}).get("us_per_step")
    return {
        "metric": "µs/decode step, LongChat layer (32 heads, 32K ctx, 2048-token "
                  "budget) as 1, 2 or 4 head groups, serial or parallel graph branches",
        "value": one, "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (as longchat; each head group its own caches)",
        "config": {"workload": "longchat_head_groups", "groups": [1, 2, 4],
                   "rotating_caches": rot, "variants": variants},
        "timing": "each variant: back-to-back replays of one HIP graph holding one "
                  "step on each rotating cache, HIP events around each replay",
        "results": out, "gpu": torch.cuda.get_device_name(0)}


def bench_host_kv(args, torch, qa, synth):
    """The LongChat layer with its K/V pools in pinned host memory: metadata,
    scores and selection stay in HBM, and attention reads only the kept
    pages over the host link ("Guide to Quest": the cache stays in host or
    device memory and only the critical pages are loaded)."""
    rot = 2
    wls = [synth.longchat_layer_workload(seed=1 + 1000 * i) for i in range(rot)]
    insts = [make_layer(qa, synth, wl) for wl in wls]
    for c in insts:                      # move the pools to the host
        c["k_pool"], c["v_pool"] = qa.host_pool_like(c["k_pool"]), \
            qa.host_pool_like(c["v_pool"])
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    kv = insts[0]["kv"]
    k = wls[0].k_pages
    sm = 1.0 / math.sqrt(128)
    steps = [qa.SparseDecodeStep(kv, k, sm) for _ in range(rot)]
    denses = [qa.DenseDecode(kv, sm) for _ in range(rot)]

    def step_call(i):
        c = insts[i]
        steps[i](c["q"], c["k_pool"], c["v_pool"], c["kmin"], c["kmax"],
                 c["page_table"], c["seq_lens"])

    def dense_call(i):
        c = insts[i]
        denses[i](c["q"], c["k_pool"], c["v_pool"], c["page_table"], c["seq_lens"])

    for i in range(rot):
        step_call(i)
        dense_call(i)
    torch.cuda.synchronize()
    us = graph_batch(torch, step_call, rot, 10, min_replays=3, warm=1)["mean"]
    us_dense = graph_batch(torch, dense_call, rot, 2, min_replays=2, warm=1)["mean"]
    lens = [int(x) for x in insts[0]["seq_lens"].cpu()]
    b = step_bytes(lens, kv.num_kv_heads, kv.num_q_heads, k,
                   sel=steps[0].sel.cpu().numpy())
    link_bytes = b["kv"]                 # what crosses the host link
    dense_link = sum(L * kv.num_kv_heads * 2 * 128 * 2 for L in lens)
    # the link's read ceiling: the streaming probe over pinned host memory
    buf = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    buf.fill_(1)
    hbuf = qa.HostPool(buf)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    qa.quest_stream_read_probe(hbuf, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        qa.quest_stream_read_probe(hbuf, sink)
    e1.record(stream)
    torch.cuda.synchronize()
    link_ceiling = (1 << 30) * 3 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    link_gbps = link_bytes / (us * 1e-6) / 1e9
    return {
        "metric": "µs/decode step with K/V in pinned host memory, 32 heads, "
                  "32K ctx, 2048-token budget",
        "value": round(us, 3), "unit": "us/step", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (as longchat); K/V pools in pinned host memory, "
                "metadata in HBM",
        "config": {"workload": "longchat7b_layer_decode_host_kv", "batch": 1,
                   "q_heads": 32, "kv_heads": 32, "ctx": 32768,
                   "budget_tokens": 2048, "rotating_caches": rot},
        "link_bytes_per_step": int(link_bytes),
        "link_GBps": round(link_gbps, 2),
        "link_read_ceiling_GBps": round(link_ceiling, 2),
        "roofline": {"bound": "host link", "achieved": round(link_gbps, 2),
                     "peak": round(link_ceiling, 2), "unit": "GB/s",
                     "frac": round(link_gbps / link_ceiling, 4), "traffic": None,
                     "kernel": "whole step (kept K/V read from host memory)"},
        "dense_us_per_step": round(us_dense, 3),
        "dense_link_bytes_per_step": int(dense_link),
        "speedup_vs_dense": round(us_dense / us, 3),
        "gpu": torch.cuda.get_device_name(0)}


def extra_workloads(args, torch, qa, synth):
    """The other workloads of the pages at their real sizes, each timed by
    the same protocol (no CPU leg): the ragged batch, the 32-layer GQA step
    and two sweep points.  Each carries its bytes and its roofline."""
    ex = {}
    for name, fn in (
            ("sweep_32k_2048", lambda: sweep_point(args, torch, qa, synth, 32768, 2048)),
            ("sweep_128k_256", lambda: sweep_point(args, torch, qa, synth, 131072, 256)),
            ("ragged_batch", lambda: bench_ragged(args, torch, qa, synth, full=False)),
            ("gqa_multistep", lambda: bench_gqa_multistep(args, torch, qa, synth,
                                                          full=False))):
        t0 = time.perf_counter()
        ex[name] = fn()
        ex[name]["bench_seconds"] = round(time.perf_counter() - t0, 1)
        print(json.dumps({"progress": name, "us_per_step": ex[name]["us_per_step"]}),
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    return ex


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
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": (f"{reps} oracle decode steps over {len(heads)} of 32 heads "
                       f"of one 32K-context layer (estimate + Top-K + sparse "
                       f"attention, float64, 1 thread), {el:.1f} s, scaled x"
                       f"{gpu['kv'].num_q_heads // len(heads)} to 32 heads")}



def _timed_loop(fn, budget_s):
    """Call fn() until budget_s seconds have passed: (calls, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def _oracle_worker(task):
    """One process of the all-cores oracle leg: the step on its kv-heads of
    the layer saved under `path` (.npy files), one thread, repeated for
    budget_s seconds.  Returns (steps, seconds, kv-heads)."""
    path, heads, group, k_pages, sm, S, budget_s = task
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import quest_oracle as O

    def ld(name, index=None):
        a = np.load(os.path.join(path, name + ".npy"), mmap_mode="r")
        return np.asarray(a if index is None else a[index], dtype=np.float64)

    qh = [g * group + i for g in heads for i in range(group)]
    q = ld("q", (slice(None), qh))
    kp = ld("k_pool", (slice(None), heads))
    vp = ld("v_pool", (slice(None), heads))
    pt = ld("page_table").astype(np.int64)
    lens = ld("seq_lens").astype(np.int64)
    with threadpool_limits(limits=1):
        kmin, kmax = O.page_meta(kp, pt, lens, S)
        reps, el = _timed_loop(
            lambda: O.decode_step(q, kp, vp, kmin, kmax, pt, lens, k_pages, sm, S),
            budget_s)
    return reps, el, len(heads)


def cpu_baseline_all_cores(gpu, budget_s):
    """The oracle's step on every kv-head of the same layer, one process
    per host core (at most 16), each single-threaded over its share of the
    heads; the per-process rates add up to the step rate.  The processes
    start fresh interpreters (spawn) and read the layer from .npy files."""
    import multiprocessing
    import tempfile

    import numpy as np
    import torch

    c, kv = gpu["insts"][0], gpu["kv"]
    H = kv.num_kv_heads
    cores = max(1, min(len(os.sched_getaffinity(0)), 16, H))
    groups = [list(range(H))[i::cores] for i in range(cores)]
    with tempfile.TemporaryDirectory(prefix="quest_oracle_") as tmp:
        for name in ("q", "k_pool", "v_pool", "page_table", "seq_lens"):
            t = c[name].cpu()
            if t.dtype == torch.bfloat16:
                t = t.float()
            np.save(os.path.join(tmp, name + ".npy"), t.numpy())
        tasks = [(tmp, g, kv.num_q_heads // H, gpu["k_pages"], gpu["sm"],
                  kv.page_size, budget_s) for g in groups]
        with multiprocessing.get_context("spawn").Pool(len(groups)) as pool:
            res = pool.map(_oracle_worker, tasks)
    rate = sum(reps * h / el for reps, el, h in res)   # kv-head steps per second
    return {"value": round(H / rate * 1e6, 1), "unit": "us/step",
            "cores": len(groups), "kind": "oracle",
            "sample": (f"all {H} kv-heads of the same layer, {len(groups)} "
                       f"single-threaded processes of {budget_s:.0f} s each "
                       f"({sum(r for r, _, _ in res)} head-group steps); the "
                       f"processes' rates summed")}


def cpu_baseline_ragged(gpu, budget_s, heads=(0, 1, 2, 3)):
    """The oracle's step on the two requests of the batch whose lengths are
    nearest its mean, 4 of the 32 heads, one thread; scaled to the whole
    batch by (request, kv-head) units."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import quest_oracle as O

    c, kv = gpu["insts"][0], gpu["kv"]
    S, H = kv.page_size, kv.num_kv_heads
    G = kv.num_q_heads // H
    lens_all = c["seq_lens"].cpu().numpy().astype(np.int64)
    pt_all = c["page_table"].cpu().numpy().astype(np.int64)
    reqs = sorted(np.argsort(np.abs(lens_all - lens_all.mean()))[:2].tolist())
    pages = [pt_all[b, :-(-int(lens_all[b]) // S)] for b in reqs]
    idx = torch.from_numpy(np.concatenate(pages)).to(c["k_pool"].device)
    f64 = lambda t: t.float().cpu().to(torch.float64).numpy()
    hs = list(heads)
    kp = f64(c["k_pool"][idx][:, hs])
    vp = f64(c["v_pool"][idx][:, hs])
    q = f64(c["q"][reqs][:, [g * G + i for g in hs for i in range(G)]])
    pt = np.zeros((len(reqs), max(len(p) for p in pages)), dtype=np.int64)
    off = 0
    for i, p in enumerate(pages):
        pt[i, :len(p)] = np.arange(off, off + len(p))
        off += len(p)
    lens = lens_all[reqs]
    with threadpool_limits(limits=1):
        kmin, kmax = O.page_meta(kp, pt, lens, S)
        reps, el = _timed_loop(
            lambda: O.decode_step(q, kp, vp, kmin, kmax, pt, lens, gpu["k_pages"],
                                  gpu["sm"], S), budget_s)
    scale = (len(lens_all) * H) / (len(reqs) * len(hs))
    return {"value": round(el / reps * scale * 1e6, 1), "unit": "us/step",
            "cores": 1, "kind": "oracle",
            "sample": (f"{reps} oracle decode steps over requests {reqs} "
                       f"(lengths {lens.tolist()}, batch mean "
                       f"{lens_all.mean():.0f}) x {len(hs)} of {H} heads, "
                       f"float64, 1 thread, {el:.1f} s, scaled x{scale:.0f} "
                       f"by (request, kv-head) units")}


def cpu_baseline_multistep(layers, wl, budget_s, heads=(0, 1)):
    """The oracle on one dense and one sparse layer, 2 of the 8 kv-heads
    (their 8 query heads), the first two decode steps (append, then dense
    attention or the sparse step), one thread, repeated from the same
    starting state; scaled to the 32-layer step of all 8 kv-heads."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import quest_oracle as O

    S = wl.page_size
    G = wl.num_q_heads // wl.num_kv_heads
    hs = list(heads)
    qh = [g * G + i for g in hs for i in range(G)]
    f64 = lambda t: t.float().cpu().to(torch.float64).numpy()
    nsteps = 2
    L0 = np.array(wl.seq_lens, dtype=np.int64)
    sm = 1.0 / math.sqrt(wl.head_dim)
    legs = {}
    for name, layer in (("dense", 0), ("sparse", wl.dense_layers)):
        st = layers[layer]
        c = st["c"]
        kp, vp = f64(c["k_pool"][:, hs]), f64(c["v_pool"][:, hs])
        pt = c["page_table"].cpu().numpy().astype(np.int64)
        kmin, kmax = O.page_meta(kp, pt, L0, S)   # the boxes before the first append
        q = [f64(st["q"][s][:, qh]) for s in range(nsteps)]
        kn = [f64(st["k_new"][s][:, hs]) for s in range(nsteps)]
        vn = [f64(st["v_new"][s][:, hs]) for s in range(nsteps)]
        legs[name] = (layer, kp, vp, kmin, kmax, pt, q, kn, vn)
    spent = {"dense": 0.0, "sparse": 0.0}
    reps = 0
    t_start = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t_start < budget_s:
            for name, (layer, kp, vp, kmin, kmax, pt, q, kn, vn) in legs.items():
                state = [a.copy() for a in (kp, vp, kmin, kmax)]   # untimed
                t0 = time.perf_counter()
                for s in range(nsteps):
                    O.layer_step(layer, wl.dense_layers, q[s], *state, pt,
                                 L0 + s + 1, kn[s], vn[s], wl.k_pages, sm, S)
                spent[name] += time.perf_counter() - t0
            reps += 1
    per_layer = {n: spent[n] / (reps * nsteps) for n in spent}
    scale = wl.num_kv_heads / len(hs)
    us = (wl.dense_layers * per_layer["dense"] +
          (wl.layers - wl.dense_layers) * per_layer["sparse"]) * scale * 1e6
    return {"value": round(us, 1), "unit": "us/step", "cores": 1, "kind": "oracle",
            "sample": (f"one dense and one sparse layer, kv-heads {hs} of "
                       f"{wl.num_kv_heads} ({len(qh)} query heads), the first "
                       f"{nsteps} decode steps, replayed {reps} times from the "
                       f"same start (float64, 1 thread; {per_layer['dense'] * 1e3:.1f} "
                       f"and {per_layer['sparse'] * 1e3:.1f} ms per layer-step); "
                       f"scaled to {wl.dense_layers} dense + "
                       f"{wl.layers - wl.dense_layers} sparse layers and x{scale:.0f} "
                       f"kv-heads")}

# ------------------------------------------------------------- counters

def _counter_medians(path):
    """Median counter value per kernel (short name) over its dispatches."""
    vals = {}
    for f in glob.glob(os.path.join(path, "*counter_collection.csv")):
        for row in csv.DictReader(open(f)):
            n = row["Kernel_Name"]
            m = re.search(r"quest::\(anonymous namespace\)::(\w+)", n)
            key = m.group(1) if m else ("copy" if "copy" in n.lower() else None)
            if key:
                vals.setdefault(key, []).append(float(row["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}, \
        {k: len(v) for k, v in vals.items()}


def pmc_summary(d, copy_mib):
    """Markdown: calibrated FETCH_SIZE + WRITE_SIZE bytes per launch."""
    fetch, nf = _counter_medians(os.path.join(d, "fetch"))
    write, _ = _counter_medians(os.path.join(d, "write"))
    cfetch, _ = _counter_medians(os.path.join(d, "cfetch"))
    cwrite, _ = _counter_medians(os.path.join(d, "cwrite"))
    copy_kib = copy_mib * 1024
    f_scale = copy_kib / cfetch["copy"]
    w_scale = copy_kib / cwrite["copy"]
    out = ["| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | "
           "calibrated bytes |", "|---|---|---|---|---|"]
    per_kernel = {}
    for k in sorted(fetch):
        if k == "copy" or k not in write:
            continue
        b = (fetch[k] * f_scale + write[k] * w_scale) * 1024
        per_kernel[k] = b
        out.append(f"| {k} | {nf[k]} | {fetch[k]:.1f} | {write[k]:.1f} | {b:.0f} |")
    calls = ["", "| kernel | HBM bytes per launch | sources digest |", "|---|---|---|"]
    for kern, srcs in KERNELS.items():
        if kern in per_kernel:
            calls.append(f"| {kern} | {per_kernel[kern]:.0f} | {sources_digest(srcs)} |")
    head = [f"Copy calibration ({copy_mib} MiB read + {copy_mib} MiB written "
            f"by one device copy): FETCH_SIZE reads {cfetch['copy']:.1f} KiB "
            f"(scale x{f_scale:.4f}), WRITE_SIZE {cwrite['copy']:.1f} KiB "
            f"(scale x{w_scale:.4f}).", ""]
    return "\n".join(head + out + calls) + "\n"


def counter_table(d):
    """Markdown: the median of each counter per kernel and grid over its
    dispatches, from rocprofv3 --pmc CSVs under d (raw counts, uncalibrated)."""
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            m = re.search(r"quest::\(anonymous namespace\)::(\w+)(<[^(]*>)?", row["Kernel_Name"])
            if not m:
                continue
            key = (m.group(1) + (m.group(2) or ""), row.get("Grid_Size", "?"))
            vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(
                float(row["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    out = ["| kernel | grid | dispatches | " + " | ".join(names) + " |",
           "|---|---|---|" + "---|" * len(names)]
    for (k, grid), v in sorted(vals.items()):
        n = max(len(x) for x in v.values())
        out.append(f"| `{k}` | {grid} | {n} | " + " | ".join(
            f"{statistics.median(v[c]):.0f}" if c in v else "" for c in names) + " |")
    return "\n".join(out) + "\n"


STEP_KERNELS = ("estimate_kernel", "topk_kernel", "topk_attn_kernel", "attn_split_kernel",
                "attn_merge_kernel", "attn_merge_wide_kernel")


def trace_summary(d):
    """Markdown: per-kernel dispatch count, mean and median duration (ns)
    and grid from rocprofv3 --kernel-trace CSVs under d."""
    rows, spans = {}, []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            n = row["Kernel_Name"]
            m = re.search(r"quest::\(anonymous namespace\)::(\w+)(<[^(]*>)?", n)
            if not m:
                continue
            key = (m.group(1) + (m.group(2) or ""),
                   f"{row.get('Grid_Size_X', row.get('Grid_Size', '?'))}x"
                   f"{row.get('Grid_Size_Y', '1')}/{row.get('Workgroup_Size_X', '?')}")
            t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
            rows.setdefault(key, []).append(t1 - t0)
            if m.group(1) in STEP_KERNELS:
                spans.append((t0, t1))
    out = ["| kernel | grid (threads x, y / workgroup) | dispatches | mean ns | median ns |",
           "|---|---|---|---|---|"]
    for (k, grid), v in sorted(rows.items(), key=lambda kv: -statistics.mean(kv[1])):
        out.append(f"| `{k}` | {grid} | {len(v)} | {statistics.mean(v):.0f} | "
                   f"{statistics.median(v):.0f} |")
    # concurrency of the step kernels: the sum of their durations over the
    # union of their busy intervals (1.0: never two at once)
    iv = sorted(spans)
    busy, cur_s, cur_e = 0, None, None
    for a, b in iv:
        if cur_e is None or a > cur_e:
            if cur_e is not None:
                busy += cur_e - cur_s
            cur_s, cur_e = a, b
        else:
            cur_e = max(cur_e, b)
    if cur_e is not None:
        busy += cur_e - cur_s
    total = sum(b - a for a, b in iv)
    if busy:
        out += ["", f"Step kernels (estimate, Top-K, attention, merge): {total / 1e3:.1f} us "
                f"of durations over {busy / 1e3:.1f} us busy, concurrency "
                f"{total / busy:.2f}."]
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="longchat",
                    choices=["longchat", "gqa_multistep", "ragged", "sweep",
                             "gqa_union", "page32", "host_kv", "head_groups"])
    ap.add_argument("--select", default="auto",
                    choices=["auto", "attention", "separate"],
                    help="where the sparse step runs its Top-K (SparseDecodeStep)")
    ap.add_argument("--rotate", type=int, default=16,
                    help="independent caches the steps cycle through (16: "
                         "1 GiB of touched bytes per pass, 4x the Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cpu-all-cores", action="store_true",
                    help="skip the oracle timed on every kv-head with one "
                         "process per host core (headline workload)")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline only: skip the ragged batch, the 32-layer "
                         "GQA step and the sweep points")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times "
                         "(calibrates the FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="only summarise rocprofv3 counter CSVs under DIR")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="only summarise rocprofv3 --kernel-trace CSVs under DIR")
    ap.add_argument("--hg-variants", default="serial,parallel",
                    help="head_groups workload: which issue orders to time")
    ap.add_argument("--counter-table", metavar="DIR",
                    help="only tabulate rocprofv3 --pmc counters under DIR per kernel")
    ap.add_argument("--copy-mib", type=int, default=512,
                    help="size the --copy-probe runs used (for --pmc-summary)")
    args = ap.parse_args()
    if args.trace_summary:
        sys.stdout.write(trace_summary(args.trace_summary))
        return
    if args.pmc_summary:
        sys.stdout.write(pmc_summary(args.pmc_summary, args.copy_mib))
        return
    if args.counter_table:
        sys.stdout.write(counter_table(args.counter_table))
        return
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
        print("bench.py measures one GPU only: the library has no multi-GPU "
              "path (the decode step would shard over (request, kv-head) "
              "units with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    import query_aware_kv_amd as qa
    import synth

    fn = {"longchat": bench_longchat, "gqa_multistep": bench_gqa_multistep,
          "ragged": bench_ragged, "sweep": bench_sweep,
          "gqa_union": bench_gqa_union, "page32": bench_page32,
          "host_kv": bench_host_kv, "head_groups": bench_head_groups}[args.workload]
    print(json.dumps(fn(args, torch, qa, synth)), flush=True)


if __name__ == "__main__":
    main()
