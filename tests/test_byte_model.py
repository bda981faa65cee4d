"""The benchmark's algorithmic byte model against the figures the pages and
the arithmetic fix.

- "The Memory Bandwidth Bottleneck of Long-Context Decoding" (Guide to
  Quest) prices decode attention by the K and V bytes it must load, and
  "Quest: Query-Aware Sparsity for Efficient Long-Context LLM Inference"
  (paper summary), Summary, puts a 7B model's KV cache at 32K tokens at
  about 16 GB (32 layers, 32 heads, head dim 128, fp16).
- "Guide to Quest", Best Practices 1: the metadata is 2 vectors per page,
  2/S of the page's K (12.5% at 16-token pages, 6.25% at 32).
- Reading the bounds of every page plus K/V of k of n pages moves
  n/16 + k page-equivalents of K+V, so the ideal speedup over dense is
  16 n / (n + 16 k): 8.0x at 32K context and a 2048-token budget.
"""
import json
import os

import pytest

import bench

pytestmark = pytest.mark.filterwarnings("ignore")

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "byte_model.json")))


def test_longchat_layer_bytes():
    b = bench.step_bytes([32768], 32, 32, 128)
    assert b["meta"] == 32 * 2048 * 2 * 128 * 2 == 32 * 2**20
    assert b["kv"] == 32 * 128 * 16 * 2 * 128 * 2 == 32 * 2**20
    assert b["q"] == 32 * 128 * 2 and b["out"] == 32 * 128 * 4
    assert b["table"] == 2048 * 4
    assert b["total"] == 67_141_632


def test_kv_cache_of_a_7b_model_at_32k_is_16_gib():
    g = GOLDEN
    assert bench.kv_cache_bytes(g["layers"], g["heads"], g["head_dim"], g["ctx"],
                                g["bytes_per_elem"]) == g["kv_cache_bytes"] == 16 * 2**30


@pytest.mark.parametrize("S", [16, 32])
def test_metadata_fraction_of_k(S):
    frac = GOLDEN["meta_fraction_of_k"][str(S)]
    L = 4096
    n = L // S
    meta = bench.step_bytes([L], 1, 1, 1, page_size=S)["meta"]
    k_bytes = n * S * 128 * 2
    assert meta / k_bytes == frac


def test_ideal_speedup_at_32k_budget_2048():
    sparse = bench.step_bytes([32768], 32, 32, 128)
    dense = bench.dense_bytes([32768], 32, 32)
    kv_only = (sparse["meta"] + sparse["kv"]) / (dense - 32 * 128 * 6 - 2048 * 4)
    assert abs(1 / kv_only - 16 * 2048 / (2048 + 16 * 128)) < 1e-12
    assert abs(1 / kv_only - 8.0) < 1e-12


def test_partial_last_page_counts_valid_tokens_only():
    # 17 tokens: page 0 full, page 1 holds one token
    b = bench.step_bytes([17], 1, 1, 2, sel=[[[0, 1]]])
    assert b["kv"] == (16 + 1) * 2 * 128 * 2
    b = bench.step_bytes([17], 1, 1, 2, sel=[[[1, -1]]])
    assert b["kv"] == 1 * 2 * 128 * 2


def test_gqa_reads_kv_once_per_kv_head():
    """Four query heads share a kv-head: K/V bytes follow Hkv, q and out Hq."""
    b = bench.step_bytes([32768], 8, 32, 128)
    assert b["kv"] == 8 * 128 * 16 * 2 * 128 * 2
    assert b["meta"] == 8 * 2048 * 512
    assert b["q"] == 32 * 128 * 2 and b["out"] == 32 * 128 * 4


def test_kernel_bytes_split_the_step_model():
    """The per-kernel algorithmic bytes of the roofline add up to the step's
    byte model (q counted once per kernel that reads it), and the round trips
    the model leaves out are listed apart."""
    import query_aware_kv_amd as qa
    kv = qa.paged_kv(1, 32, 32, 2048, 2048, __import__("torch").float16)
    avg = bench.step_bytes([32768], 32, 32, 128)
    kb = bench.kernel_bytes(avg, kv, 128)
    est, ta, mg = (kb[n][0] for n in ("estimate_kernel", "topk_attn_kernel",
                                      "attn_merge_kernel"))
    assert est + ta + mg == avg["total"] + avg["q"]
    assert ta == 32 * 128 * 8192 + avg["q"]          # kept K/V + q
    over = kb["topk_attn_kernel"][1]
    assert over["scores_read"] == 32 * 2048 * 4 and over["sel_written"] == 32 * 128 * 4
    # 8 splits of 16 pages per row at 32 rows: 32 heads x 8 partials
    assert over["partials_written"] == 32 * 8 * 130 * 4
    assert bench.topk_attn_splits(8, 128) == 16      # 8 rows: one page per wave


def test_roofline_takes_the_slowest_kernel():
    ku = {"estimate_kernel": 8.0, "topk_attn_kernel": 12.0, "attn_merge_kernel": 1.5}
    kb = {"estimate_kernel": (33_570_816, {}),
          "topk_attn_kernel": (33_562_624, {"scores_read": 262144}),
          "attn_merge_kernel": (16384, {})}
    r = bench.roofline(ku, kb)
    assert r["kernel"] == "topk_attn_kernel" and r["kernel_us"] == 12.0
    assert abs(r["achieved"] - 33_562_624 / 12e-6 / 1e9) < 0.1
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-4
    assert r["overhead_bytes_per_launch"] == {"scores_read": 262144}
    assert r["traffic"] is None


def test_recorded_traffic_needs_its_workload_file_and_current_sources(tmp_path):
    digest = bench.sources_digest(bench.KERNELS["topk_attn_kernel"])
    f = tmp_path / "traffic.md"
    f.write_text("| kernel | HBM bytes per launch | sources digest |\n|---|---|---|\n"
                 f"| topk_attn_kernel | 36000000 | {digest} |\n"
                 "| estimate_kernel | 34000000 | 0000000000000000 |\n")
    assert bench.recorded_traffic("topk_attn_kernel", str(f)) == (36000000, digest)
    # a digest of other sources: no record
    assert bench.recorded_traffic("estimate_kernel", str(f))[0] is None
    assert bench.recorded_traffic("topk_attn_kernel", str(tmp_path / "none.md"))[0] is None
    ku = {"topk_attn_kernel": 12.0}
    kb = {"topk_attn_kernel": (33_562_624, {})}
    r = bench.roofline(ku, kb, str(f))
    assert r["traffic"] == 36000000 and digest in r["traffic_source"]
    assert bench.roofline(ku, kb)["traffic"] is None


def test_recorded_traffic_of_a_two_kernel_call_is_the_sum(tmp_path):
    d1 = bench.sources_digest(bench.KERNELS["attn_split_kernel"])
    d2 = bench.sources_digest(bench.KERNELS["attn_merge_kernel"])
    f = tmp_path / "traffic.md"
    f.write_text(f"| attn_split_kernel | 1000 | {d1} |\n| attn_merge_kernel | 24 | {d2} |\n")
    ku = {"attn_split_kernel+attn_merge_kernel": 10.0}
    kb = {"attn_split_kernel+attn_merge_kernel": (1000, {})}
    assert bench.roofline(ku, kb, str(f))["traffic"] == 1024
    f.write_text(f"| attn_split_kernel | 1000 | {d1} |\n")
    assert bench.roofline(ku, kb, str(f))["traffic"] is None
