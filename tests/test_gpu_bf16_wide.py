"""GPU parity of the 256x256-tile bf16 kernel (tile configuration kernel=2)
for the forward, dX and tgmm against the fp64 oracle, at the bf16 bar
|gpu - ref| <= 1e-3 + 2e-2 |ref| ("GEMM Kernel 性能优化十问", Q5: the backward
is unquantised bf16 with fp32 accumulation): ragged groups, empty groups,
single rows, groups spanning several 256-row items, rows past the total,
more than 64 groups, both output types, and the production shape in full."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, tile_config, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WIDE = {"kernel": 2}

CASES = [
    (1, 256, 256, [1]),
    (300, 256, 512, [100, 0, 0, 150]),
    (1000, 512, 256, [1] * 200 + [700]),
    (2000, 256, 256, [600, 0, 3, 1100, 250]),
    (777, 512, 512, [256, 255, 257]),
    (1500, 256, 256, list(np.random.default_rng(3).integers(0, 20, 70))),
]


def _gs(wl):
    return torch.from_numpy(wl.group_sizes).to(DEV)


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_forward(M, K, N, gs, out_dtype):
    wl = workloads.custom(M, K, N, gs, seed=M + K, w_std=0.05)
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, WIDE):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "wide fwd")


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dx(M, K, N, gs, out_dtype):
    wl = workloads.custom(M, K, N, gs, seed=M + 2 * K, w_std=0.05, with_dy=True)
    out = torch.full((M, K), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_DX, WIDE):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "wide dx")


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("placement", [0, 1])
def test_tgmm(M, K, N, gs, out_dtype, placement):
    wl = workloads.custom(M, K, N, gs, seed=M + 3 * K, with_dy=True)
    G = len(gs)
    out = torch.full((G, K, N), float("nan"), dtype=out_dtype, device=DEV)
    cfg = dict(WIDE, placement=placement) if placement else WIDE
    with tile_config(gmm.OP_TGMM, cfg):
        gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out=out)
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    assert not np.isnan(o).any()
    for g in range(G):
        if wl.group_sizes[g] == 0:
            assert (o[g] == 0).all()
    assert_bf16_parity(o, ref, "wide tgmm")


def test_production_shape_full():
    """M=65536, G=256 with the Zipf routing: every dX row and every tgmm expert."""
    wl = workloads.make("full", seed=0, with_dy=True)
    x, dy, w, g = wl.x.to(DEV), wl.dy.to(DEV), wl.w.to(DEV), _gs(wl)
    with tile_config(gmm.OP_DX, WIDE):
        dx = gmm.gmm_bf16_dx(dy, w, g)
    with tile_config(gmm.OP_TGMM, WIDE):
        dw = gmm.tgmm_bf16(x, dy, g)
    with tile_config(gmm.OP_BF16_FWD, WIDE):
        y = gmm.gmm_bf16_fwd(x, w, g)
    xs, dys, ws = workloads.as_f32(wl.x), workloads.as_f32(wl.dy), workloads.as_f32(wl.w)
    assert_bf16_parity(to_np64(dx), oracle.gmm_dx(dys, ws, wl.group_sizes), "wide dx full")
    assert_bf16_parity(to_np64(dw), oracle.tgmm(xs, dys, wl.group_sizes), "wide tgmm full")
    assert_bf16_parity(to_np64(y), oracle.gmm(xs, ws, wl.group_sizes), "wide fwd full")
