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
