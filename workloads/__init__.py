"""Seeded synthetic inputs for the grouped-matmul workloads.

This module only draws random inputs (routing counts and tensor values); it
holds none of the method's arithmetic, so both the oracle side and the GPU
side of every test use it.  Every array comes from
``numpy.random.default_rng([seed, stream])`` with one stream per tensor, and
bf16 tensors are rounded from fp32 with round-to-nearest-even (torch's CPU
cast).  Shapes and distributions follow the pages' production and
development shapes ("GEMM Kernel 性能优化十问", Q6: M = batch x seq x top-k
= 2 x 4096 x 8, K = 2048, N = 512, G = 256, and the EP=8 shard M = 8192,
G = 32; the wo layer swaps K and N).
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

STREAM_ROUTING, STREAM_LHS, STREAM_RHS, STREAM_DY, STREAM_UP = 0, 1, 2, 3, 4


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


# ------------------------------------------------------------ routing -------

def topk_routing_counts(tokens: int, experts: int, top_k: int, seed: int,
                        log_popularity: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-expert row counts after top-k routing of `tokens` tokens.

    Logits are i.i.d. N(0,1) per (token, expert); with `log_popularity`
    they are log p_e + Gumbel(0,1) instead, which draws k distinct experts
    without replacement with probability proportional to p.  Each token
    takes its k largest logits; the counts are the bincount over experts.
    """
    r = rng(seed, STREAM_ROUTING)
    if log_popularity is None:
        logits = r.standard_normal((tokens, experts), dtype=np.float32)
    else:
        logits = log_popularity[None, :] + r.gumbel(size=(tokens, experts)).astype(np.float32)
    top = np.argpartition(-logits, top_k - 1, axis=1)[:, :top_k]
    return np.bincount(top.reshape(-1), minlength=experts).astype(np.int32)


def zipf_log_popularity(experts: int, s: float, seed: int) -> np.ndarray:
    """log p_e for p_e proportional to (rank_e + 1)^-s over a seeded permutation."""
    r = rng(seed, STREAM_ROUTING + 10)
    rank = r.permutation(experts)
    return (-s * np.log(rank + 1.0)).astype(np.float32)


def skew_counts(counts: np.ndarray, total: int, empty: int, heavy_frac: float,
                seed: int) -> np.ndarray:
    """Force `empty` experts to 0 rows and one expert to round(heavy_frac*total)
    rows; the others share the rest in proportion to `counts` (largest
    remainder).  Expert choice is seeded."""
    r = rng(seed, STREAM_ROUTING + 20)
    G = counts.size
    pick = r.choice(G, size=empty + 1, replace=False)
    empties, heavy = pick[:empty], pick[empty]
    out = np.zeros(G, dtype=np.int64)
    out[heavy] = int(round(heavy_frac * total))
    rest = [g for g in range(G) if g not in set(pick.tolist())]
    remain = total - out[heavy]
    w = counts[rest].astype(np.float64)
    ideal = w / w.sum() * remain
    base = np.floor(ideal).astype(np.int64)
    short = remain - base.sum()
    order = np.argsort(-(ideal - base), kind="stable")
    base[order[:short]] += 1
    out[rest] = base
    assert out.sum() == total and (out[empties] == 0).all()
    return out.astype(np.int32)


# ------------------------------------------------------------ configs -------

@dataclass
class Workload:
    name: str
    M: int
    K: int
    N: int
    G: int
    group_sizes: np.ndarray          # int32 [G]
    x: torch.Tensor                  # LHS [M,K] (bf16 or fp32, CPU)
    w: torch.Tensor                  # RHS [G,K,N] (bf16 or fp32, CPU)
    dy: Optional[torch.Tensor] = None  # upstream gradient [M,N] (bf16, CPU)
    out_dtype: torch.dtype = torch.bfloat16


CONFIGS = {
    # tiny FP8 forward: multinomial groups, fp32 LHS and RHS, fp32 output
    "tiny": dict(M=512, G=4, K=256, N=256),
    # dev wi layer (EP=8 shard): top-8 of 1024 tokens over 32 experts
    "wi": dict(M=8192, G=32, K=2048, N=512),
    # dev wo layer: K and N swapped, 2 empty experts, one with 30% of rows
    "wo": dict(M=8192, G=32, K=512, N=2048),
    # backward at the wi shape: tgmm and dX, all inputs bf16 N(0,1)
    "bwd": dict(M=8192, G=32, K=2048, N=512),
    # full production wi layer on one GPU: Zipf(1.1) top-8 of 8192 tokens
    "full": dict(M=65536, G=256, K=2048, N=512),
    # wi layer with the gate and up projections fused: weights [G,K,2x512],
    # gate columns first (the wi layer's own weights), then the up columns
    "wi_gate_up": dict(M=8192, G=32, K=2048, N=1024),
}


def make(name: str, seed: int = 0, with_dy: Optional[bool] = None) -> Workload:
    cfg = CONFIGS[name]
    M, G, K, N = cfg["M"], cfg["G"], cfg["K"], cfg["N"]
    if name == "tiny":
        p = np.full(G, 1.0 / G)
        gs = rng(seed, STREAM_ROUTING).multinomial(M, p).astype(np.int32)
        x = torch.from_numpy(rng(seed, STREAM_LHS).standard_normal((M, K), dtype=np.float32))
        w = torch.from_numpy(
            (rng(seed, STREAM_RHS).standard_normal((G, K, N), dtype=np.float32) * np.float32(0.05)))
        wl = Workload(name, M, K, N, G, gs, x, w, out_dtype=torch.float32)
        if with_dy:
            wl.dy = to_bf16(rng(seed, STREAM_DY).standard_normal((M, N), dtype=np.float32))
        return wl
    if name in ("wi", "bwd", "wi_gate_up"):
        gs = topk_routing_counts(M // 8, G, 8, seed)
    elif name == "wo":
        gs = skew_counts(topk_routing_counts(M // 8, G, 8, seed), M, 2, 0.3, seed)
    elif name == "full":
        gs = topk_routing_counts(M // 8, G, 8, seed, zipf_log_popularity(G, 1.1, seed))
    else:
        raise KeyError(name)
    assert int(gs.sum()) == M
    x = to_bf16(rng(seed, STREAM_LHS).standard_normal((M, K), dtype=np.float32))
    w_std = 1.0 if name == "bwd" else 0.02
    if name == "wi_gate_up":   # gate = the wi layer's weights; up from its own stream
        gate = rng(seed, STREAM_RHS).standard_normal((G, K, N // 2), dtype=np.float32)
        up = rng(seed, STREAM_UP).standard_normal((G, K, N // 2), dtype=np.float32)
        w = to_bf16(np.concatenate([gate, up], axis=2) * np.float32(w_std))
    else:
        w = to_bf16(rng(seed, STREAM_RHS).standard_normal((G, K, N), dtype=np.float32) * np.float32(w_std))
    wl = Workload(name, M, K, N, G, gs, x, w)
    if with_dy is None:
        with_dy = name in ("bwd", "full")
    if with_dy:
        wl.dy = to_bf16(rng(seed, STREAM_DY).standard_normal((M, N), dtype=np.float32))
    return wl


def custom(M: int, K: int, N: int, group_sizes, seed: int = 0,
           x_std: float = 1.0, w_std: float = 0.05, dtype=torch.bfloat16,
           with_dy: bool = False) -> Workload:
    """Small ad-hoc workload with given group sizes (edge-case tests)."""
    gs = np.asarray(group_sizes, dtype=np.int32)
    G = gs.size
    xf = rng(seed, STREAM_LHS).standard_normal((M, K), dtype=np.float32) * np.float32(x_std)
    wf = rng(seed, STREAM_RHS).standard_normal((G, K, N), dtype=np.float32) * np.float32(w_std)
    if dtype == torch.bfloat16:
        x, w = to_bf16(xf), to_bf16(wf)
    else:
        x, w = torch.from_numpy(xf), torch.from_numpy(wf)
    wl = Workload("custom", M, K, N, G, gs, x, w,
                  out_dtype=torch.float32 if dtype == torch.float32 else torch.bfloat16)
    if with_dy:
        wl.dy = to_bf16(rng(seed, STREAM_DY).standard_normal((M, N), dtype=np.float32))
    return wl


def as_f32(t: torch.Tensor) -> np.ndarray:
    """Exact fp32 widening of a CPU tensor, as numpy."""
    return t.float().numpy()
