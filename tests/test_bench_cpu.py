"""bench.py's reporting on the CPU: the per-stage summary and the headline
roofline of every workload, computed from synthetic stage times (no GPU), so
that a workload run as the main --workload cannot fail after its GPU work."""
import math

import pytest

import bench
from datagen.configs import WORKLOADS

STAGES = ["K0 indexer_prologue", "K0m mla_prologue", "K1q quant_fp8 q_idx", "K1k quant_fp8 k_idx",
          "K1 index_scores", "K2 topk", "K3 sparse_attn_prefill", "K4 sparse_attn_decode",
          "K5 swa_attn chunk", "K5 swa_attn chunk L1", "K5 swa_attn chunk L2",
          "D K1 index_scores", "D K2 topk", "D K4 sparse_attn_decode", "D K5 swa_attn",
          "D K5 swa_attn L1", "D K5 swa_attn L2"]


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_summary_and_headline_roofline(name):
    wl = WORKLOADS[name]
    ps = {s: {"mean_us": 100.0, "min_us": 100.0, "median_us": 100.0} for s in STAGES}
    r = bench.summarize(wl, ps, 1.0)
    assert r["workload"] == name
    roof = bench.headline_roofline(wl, ps)
    assert roof["bound"] in ("mfma", "hbm") and roof["unit"] in ("TFLOP/s", "GB/s")
    assert math.isfinite(roof["frac"]) and roof["frac"] > 0
    assert roof["achieved"] == pytest.approx(roof["frac"] * roof["peak"])
