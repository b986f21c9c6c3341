"""Seeded input generators: shapes, group-size structure and determinism."""
import numpy as np
import torch

import workloads


def test_tiny_shapes_and_sum():
    wl = workloads.make("tiny", seed=0)
    assert wl.x.shape == (512, 256) and wl.x.dtype == torch.float32
    assert wl.w.shape == (4, 256, 256)
    assert wl.group_sizes.sum() == 512 and wl.group_sizes.size == 4
    assert wl.out_dtype == torch.float32


def test_routing_top8_counts():
    gs = workloads.topk_routing_counts(1024, 32, 8, seed=0)
    assert gs.sum() == 8192 and gs.size == 32 and (gs <= 1024).all()
    gs2 = workloads.topk_routing_counts(1024, 32, 8, seed=0)
    assert np.array_equal(gs, gs2)
    assert not np.array_equal(gs, workloads.topk_routing_counts(1024, 32, 8, seed=1))


def test_wo_skew_structure():
    gs = workloads.skew_counts(workloads.topk_routing_counts(1024, 32, 8, 0), 8192, 2, 0.3, 0)
    assert gs.sum() == 8192
    assert (gs == 0).sum() >= 2
    assert gs.max() == round(0.3 * 8192)


def test_zipf_full_routing_is_skewed():
    lp = workloads.zipf_log_popularity(256, 1.1, 0)
    gs = workloads.topk_routing_counts(8192, 256, 8, 0, lp)
    assert gs.sum() == 65536 and gs.size == 256
    assert gs.max() > 10 * np.median(gs)       # heavy head
    assert gs.max() <= 8192                    # one expert at most once per token


def test_bf16_rounding_is_rne():
    a = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8)], np.float32)
    b = workloads.to_bf16(a).float().numpy()
    assert b.tolist() == [1.0, 1.0 + 2 ** -6, -1.0]


def _golden():
    import os
    vals = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "shapes_and_tolerances.txt")
    for line in open(path, encoding="utf-8"):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (p.strip() for p in line.split("="))
            vals[k] = float(v)
    return vals


def test_shapes_follow_the_pages_derivation():
    """Production and development shapes ("GEMM Kernel 性能优化十问", Q6)."""
    g = _golden()
    assert g["per_device_batch"] * g["seq_len"] * g["top_k"] == g["prod_wi_M"]
    full, wi, wo = (workloads.CONFIGS[n] for n in ("full", "wi", "wo"))
    assert (full["M"], full["K"], full["N"], full["G"]) == (
        g["prod_wi_M"], g["emb_dim"], g["moe_mlp_dim"], g["num_experts"])
    assert wi["M"] == g["prod_wi_M"] / g["expert_parallel"] == g["dev_M"]
    assert wi["G"] == g["num_experts"] / g["expert_parallel"] == g["dev_G"]
    assert (wi["K"], wi["N"]) == (g["prod_wi_K"], g["prod_wi_N"])
    assert (wo["M"], wo["G"], wo["K"], wo["N"]) == (g["dev_M"], g["dev_G"], g["prod_wo_K"], g["prod_wo_N"])
    # the full workload's routing: top-8 of (2 x 4096) tokens fills every row
    wl_gs = workloads.topk_routing_counts(int(g["per_device_batch"] * g["seq_len"]), full["G"],
                                          int(g["top_k"]), 0, workloads.zipf_log_popularity(full["G"], 1.1, 0))
    assert wl_gs.sum() == full["M"]


def test_tolerances_follow_the_pages():
    """The parity bar is the pages' FP8-vs-reference check, SQNR held above
    their 'good' threshold ("GEMM Kernel 性能优化十问", Q9.2)."""
    import helpers
    g = _golden()
    assert helpers.FP8_ATOL == g["fp8_vs_ref_atol"] and helpers.FP8_RTOL == g["fp8_vs_ref_rtol"]
    assert helpers.FP8_MIN_SQNR_DB >= g["sqnr_good_db"]
    assert (g["lhs_block_rows"], g["lhs_block_cols"], g["rhs_block_rows"], g["rhs_block_cols"]) == (1, 128, 128, 128)


def test_wi_gate_up_gate_half_is_the_wi_layer():
    a = workloads.make("wi", seed=0, with_dy=False)
    b = workloads.make("wi_gate_up", seed=0, with_dy=False)
    assert np.array_equal(a.group_sizes, b.group_sizes)
    assert torch.equal(a.x, b.x)
    assert b.w.shape == (32, 2048, 1024)
    assert torch.equal(b.w[:, :, :512], a.w)
    assert not torch.equal(b.w[:, :, 512:], a.w)
