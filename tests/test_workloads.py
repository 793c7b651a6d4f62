"""The seeded workload table: shapes against the SonicMoE page's trend table, determinism, scale."""
import json
import math
import os

import torch

from mixture_experts_layer_lds_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_shapes_reproduce_trend_table_ratios():
    with open(os.path.join(GOLDEN, "sonicmoe_trend_table.json")) as f:
        rows = {r["model"]: r for r in json.load(f)["rows"]}
    for cfg, model in ((wl.BY_NAME["deepseek_v3"], "DeepSeek-V3"), (wl.BY_NAME["kimi_k2"], "Kimi K2")):
        r = rows[model]
        assert (cfg.K, cfg.E) == (r["K"], r["E"])
        assert abs(100.0 * cfg.K / cfg.E - r["active_ratio_percent"]) <= 0.005 + 1e-12
        assert abs(cfg.d / cfg.n - r["d_over_n"]) <= 0.005 + 1e-12
    mix = wl.BY_NAME["mixtral_coarse"]
    assert 100.0 * mix.K / mix.E == rows["Mixtral 8x22B"]["active_ratio_percent"]
    fg = wl.BY_NAME["fine_grained_7b"]
    assert fg.T == 32768 and fg.backward          # "microbatch 32768" kernel benchmark


def test_inputs_are_seeded_and_scaled():
    cfg = wl.small_shape(T=512, d=256, E=4, K=2, n=128, dtype="bf16", bias="zipf")
    a = wl.make_inputs(cfg)
    b = wl.make_inputs(cfg)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    assert a["X"].dtype == torch.bfloat16 and a["bias"].dtype == torch.float32
    assert abs(a["X"].float().std().item() - 1.0) < 0.02
    assert abs(a["W_gate"].float().std().item() - 1 / math.sqrt(256)) < 0.002
    assert abs(a["W_down"].float().std().item() - 1 / math.sqrt(128)) < 0.002
    assert abs(a["W_r"].float().std().item() - 0.02) < 0.001
    ranks = torch.exp(a["bias"].double() / -1.1)
    assert sorted(round(x) for x in ranks.tolist()) == [1, 2, 3, 4]
