"""Seeded random sweep of small grouped problems for the bf16 calls (forward
baseline, tgmm, dX) on the GPU against the fp64 oracle: random M, K, N, G
within each call's shape rules, the same four group-size patterns as the
FP8 sweep (uniform, one dominant group, many empty and size-1 groups,
Zipf-like), rows past the total, bf16 or fp32 output, and the library's
choice or a fixed kernel / placement.  Outputs are NaN-filled first, so an
element the call never writes fails; outputs within
|gpu - ref| <= 1e-3 + 2e-2 |ref| ("GEMM Kernel 性能优化十问", Q5: the backward
pass is unquantised bf16 with fp32 accumulation); rows past the total are
zero, and so is an empty group's weight gradient.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, tile_config, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = 24


def group_sizes(r, G, total, pattern):
    if pattern == 0:                                     # uniform routing
        gs = r.multinomial(total, np.full(G, 1.0 / G))
    elif pattern == 1:                                   # one dominant group
        p = np.full(G, 0.1 / G)
        p[r.integers(G)] += 0.9
        gs = r.multinomial(total, p / p.sum())
    elif pattern == 2:                                   # many empty and size-1 groups
        gs = np.zeros(G, np.int64)
        gs[r.choice(G, max(1, G // 3), replace=False)] = 1
        gs[int(r.integers(G))] += total
    else:                                                # Zipf-like popularity
        p = 1.0 / np.arange(1, G + 1) ** 1.1
        gs = r.multinomial(total, p / p.sum())
    return gs.astype(np.int32)


def random_problem(seed, kq, nq):
    """K a multiple of kq, N of nq (the call's shape rules)."""
    r = workloads.rng(3000 + seed, 9)
    K = kq * int(r.integers(1, 1024 // kq + 1))
    N = nq * int(r.integers(1, 768 // nq + 1))
    G = int(r.choice([1, 2, 3, 7, 16, 40]))
    gs = group_sizes(r, G, int(r.integers(1, 900)), seed % 4)
    M = int(gs.sum()) + int(r.integers(0, 70))           # rows past the total
    wl = workloads.custom(M, K, N, gs, seed=4000 + seed, w_std=float(r.choice([0.02, 0.05, 1.0])),
                          with_dy=True)
    out_dtype = torch.float32 if seed % 2 else torch.bfloat16
    return wl, out_dtype, r


def config(seed, r, op, K, N):
    """None (the library's choice), kernel 1, or kernel 3 with two LDS stages;
    a random placement where the call takes one."""
    kind = seed % 3
    if kind == 0:
        return None
    cfg = {"kernel": 1} if kind == 1 else {"kernel": 3, "depth": 2}
    if op == gmm.OP_TGMM:
        ok = [0, 1] + ([2] if ((K // 128) * (N // 128)) % 8 == 0 else [])
        cfg["placement"] = int(r.choice(ok))
    else:
        cfg["placement"] = int(r.choice([1, 2]))
    return cfg


def _case(wl, cfg):
    return "M=%d K=%d N=%d G=%d cfg=%s" % (wl.M, wl.K, wl.N, wl.G, cfg)


@pytest.mark.parametrize("seed", range(CASES))
def test_bf16_fwd_random(seed):
    wl, out_dtype, r = random_problem(seed, 64, 128)
    cfg = config(seed, r, gmm.OP_BF16_FWD, wl.K, wl.N)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, cfg):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), torch.from_numpy(wl.group_sizes).to(DEV), out=out)
    torch.cuda.synchronize()
    ref = oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all(), _case(wl, cfg)
    assert_bf16_parity(o, ref, "bf16 fwd random %d (%s)" % (seed, _case(wl, cfg)))


@pytest.mark.parametrize("seed", range(CASES))
def test_dx_random(seed):
    wl, out_dtype, r = random_problem(seed, 128, 64)
    cfg = config(seed, r, gmm.OP_DX, wl.K, wl.N)
    out = torch.full((wl.M, wl.K), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_DX, cfg):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), torch.from_numpy(wl.group_sizes).to(DEV), out=out)
    torch.cuda.synchronize()
    ref = oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all(), _case(wl, cfg)
    assert_bf16_parity(o, ref, "dx random %d (%s)" % (seed, _case(wl, cfg)))


@pytest.mark.parametrize("seed", range(CASES))
def test_tgmm_random(seed):
    wl, out_dtype, r = random_problem(seed, 128, 128)
    cfg = config(seed, r, gmm.OP_TGMM, wl.K, wl.N)
    out = torch.full((wl.G, wl.K, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_TGMM, cfg):
        gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), torch.from_numpy(wl.group_sizes).to(DEV), out=out)
    torch.cuda.synchronize()
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    for g in np.flatnonzero(wl.group_sizes == 0):
        assert (o[g] == 0).all(), "empty group %d must give exactly zero (%s)" % (g, _case(wl, cfg))
    assert_bf16_parity(o, ref, "tgmm random %d (%s)" % (seed, _case(wl, cfg)))
