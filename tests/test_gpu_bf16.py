"""GPU parity of the bf16 grouped matmuls (forward baseline, tgmm, dX) against
the fp64 oracle: |gpu - ref| <= 1e-3 + 2e-2 |ref| ("GEMM Kernel 性能优化十问",
Q5: the backward pass is unquantised bf16 with fp32 accumulation)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, tile_config, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

EDGE = [
    (1, 128, 128, [1]),
    (7, 256, 256, [3, 0, 4]),
    (129, 384, 128, [0, 129]),
    (300, 256, 384, [100, 0, 0, 150]),
    (1000, 512, 256, [1] * 200 + [800]),
    (513, 128, 256, [0, 0, 513, 0]),
    (640, 256, 128, [128, 128, 128, 128, 128]),
]


def _gs(wl):
    return torch.from_numpy(wl.group_sizes).to(DEV)


@pytest.mark.parametrize("M,K,N,gs", EDGE)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("kernel", [1, 3])
def test_bf16_fwd_edges(M, K, N, gs, out_dtype, placement, kernel):
    """placement 2: row tiles start at each group's first row; kernel 1
    register-staged, 3 load-to-LDS (its default stages)."""
    wl = workloads.custom(M, K, N, gs, seed=M + 3 * K, w_std=0.05)
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, {"kernel": kernel, "placement": placement}):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "bf16 fwd")


@pytest.mark.parametrize("M,K,N,gs", EDGE)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("kernel", [1, 3])
def test_dx_edges(M, K, N, gs, out_dtype, placement, kernel):
    wl = workloads.custom(M, K, N, gs, seed=M + 5 * K, w_std=0.05, with_dy=True)
    out = torch.full((M, K), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_DX, {"kernel": kernel, "placement": placement}):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "dx")


@pytest.mark.parametrize("M,K,N,gs", EDGE)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kernel", [1, 3])
def test_tgmm_edges(M, K, N, gs, out_dtype, kernel):
    wl = workloads.custom(M, K, N, gs, seed=M + 7 * K, with_dy=True)
    G = len(gs)
    out = torch.full((G, K, N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_TGMM, {"kernel": kernel}):
        gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out=out)
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    for g in range(G):
        if gs[g] == 0:
            assert (o[g] == 0).all(), "empty group must give exactly zero"
    assert_bf16_parity(o, ref, "tgmm")


def test_tgmm_ignores_tail_rows():
    wl = workloads.custom(300, 128, 128, [100, 150], seed=31, with_dy=True)
    x = wl.x.clone()
    x[250:] = 1e30
    a = gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out_dtype=torch.float32)
    b = gmm.tgmm_bf16(x.to(DEV), wl.dy.to(DEV), _gs(wl), out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_exact_integers_bitwise():
    """Small-integer inputs: every fp32 partial sum is exact, so fwd, dX and tgmm
    must equal the oracle bit for bit."""
    r = workloads.rng(41, 0)
    M, K, N = 300, 256, 256
    gs = np.array([120, 0, 180], np.int32)
    x = torch.from_numpy(r.integers(-8, 9, (M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(r.integers(-8, 9, (3, K, N)).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(r.integers(-8, 9, (M, N)).astype(np.float32)).to(torch.bfloat16)
    g = torch.from_numpy(gs).to(DEV)
    xf, wf, dyf = workloads.as_f32(x), workloads.as_f32(w), workloads.as_f32(dy)
    assert np.array_equal(to_np64(gmm.gmm_bf16_fwd(x.to(DEV), w.to(DEV), g, out_dtype=torch.float32)),
                          oracle.gmm(xf, wf, gs))
    assert np.array_equal(to_np64(gmm.gmm_bf16_dx(dy.to(DEV), w.to(DEV), g, out_dtype=torch.float32)),
                          oracle.gmm_dx(dyf, wf, gs))
    assert np.array_equal(to_np64(gmm.tgmm_bf16(x.to(DEV), dy.to(DEV), g, out_dtype=torch.float32)),
                          oracle.tgmm(xf, dyf, gs))


def test_bwd_config_full():
    """Backward at the wi shape (M=8192, G=32, K=2048, N=512), all bf16 N(0,1)."""
    wl = workloads.make("bwd", seed=0)
    g = _gs(wl)
    x, w, dy = wl.x.to(DEV), wl.w.to(DEV), wl.dy.to(DEV)
    xf, wf, dyf = workloads.as_f32(wl.x), workloads.as_f32(wl.w), workloads.as_f32(wl.dy)
    for out_dtype in (torch.bfloat16, torch.float32):
        dw = gmm.tgmm_bf16(x, dy, g, out_dtype=out_dtype)
        assert_bf16_parity(to_np64(dw), oracle.tgmm(xf, dyf, wl.group_sizes), "tgmm bwd")
    dx = gmm.gmm_bf16_dx(dy, w, g)
    assert_bf16_parity(to_np64(dx), oracle.gmm_dx(dyf, wf, wl.group_sizes), "dx bwd")
    y = gmm.gmm_bf16_fwd(x, w, g)
    assert_bf16_parity(to_np64(y), oracle.gmm(xf, wf, wl.group_sizes), "fwd bwd-shape")


def test_wi_bf16_baseline_full():
    wl = workloads.make("wi", seed=0, with_dy=False)
    y = gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl))
    assert_bf16_parity(to_np64(y), oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w),
                                               wl.group_sizes), "bf16 wi")


def test_tgmm_many_groups_mixed_sizes_every_group_written():
    """76 groups (more than one 64-lane scan chunk) of mixed sizes: over 2048
    rows, a few hundred, a single row, empty, and sizes one below or at a
    multiple of the 64-row reduction step.  The largest group holds more
    than four times the mean and there are 8 tiles per group, so tgmm takes
    its skewed-routing placement (tiles spread over the XCDs, groups by size
    class).  Every dW[g] must be written (the output starts as NaN), empty
    groups exactly zero, all matching the oracle; the uniform-routing
    placement is covered by the wi-shape backward test."""
    sizes = [5, 2100, 0, 130, 600, 1, 0, 2048, 127, 511, 512, 128] + [3, 70, 0, 200] * 16
    M = int(sum(sizes)) + 37
    assert max(sizes) * len(sizes) > 4 * sum(sizes)
    wl = workloads.custom(M, 512, 256, sizes, seed=97, with_dy=True)
    G = len(sizes)
    out = torch.full((G, 512, 256), float("nan"), dtype=torch.float32, device=DEV)
    gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out=out)
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    assert not np.isnan(o).any()
    for g in range(G):
        if sizes[g] == 0:
            assert (o[g] == 0).all()
    assert_bf16_parity(o, ref, "tgmm mixed sizes")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("kernel", [1, 3])
def test_dx_straddling_tiles_ragged_tail(out_dtype, placement, kernel):
    """dX over several 128-row tiles with straddling groups, a ragged tail and
    K spanning several column tiles; rows past the total are zero."""
    gs = [70, 0, 129, 200, 1, 0, 33]
    M = int(sum(gs)) + 50
    wl = workloads.custom(M, 512, 384, gs, seed=123, w_std=0.05, with_dy=True)
    out = torch.full((M, 512), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_DX, {"kernel": kernel, "placement": placement}):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(sum(gs)):] == 0).all()
    assert_bf16_parity(o, ref, "dx straddling")


@pytest.mark.parametrize("skewed", [True, False])
@pytest.mark.parametrize("kernel", [1, 3])
def test_tgmm_more_than_256_groups(skewed, kernel):
    """300 groups: tgmm's placement reads the sizes chunk by chunk from
    memory (above 256 groups), both with the skewed-routing placement (one
    group of 3000 rows, 8 tiles per group) and the default one."""
    r = workloads.rng(131, 0)
    sizes = r.integers(0, 12, 300).astype(np.int64)
    sizes[::17] = 0
    if skewed:
        sizes[211] = 3000
    else:
        sizes[211] = 20
    assert (sizes.max() * len(sizes) > 4 * sizes.sum()) == skewed
    M = int(sizes.sum()) + 5
    wl = workloads.custom(M, 512, 256, sizes.tolist(), seed=133, with_dy=True)
    G = len(sizes)
    out = torch.full((G, 512, 256), float("nan"), dtype=torch.float32, device=DEV)
    with tile_config(gmm.OP_TGMM, {"kernel": kernel}):
        gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out=out)
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    assert not np.isnan(o).any()
    for g in range(G):
        if sizes[g] == 0:
            assert (o[g] == 0).all()
    assert_bf16_parity(o, ref, "tgmm 300 groups")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_bf16_fwd_multi_round_grid(out_dtype):
    """A forward grid of more than two workgroups per CU (4096 rows, 2048
    columns: 624 blocks), which takes kernel 1's variant compiled for three
    resident workgroups per CU; straddling groups, an empty one and a ragged
    tail."""
    gs = [700, 0, 1313, 1, 1000, 999]
    M = int(sum(gs)) + 83
    wl = workloads.custom(M, 256, 2048, gs, seed=211, w_std=0.05)
    out = torch.full((M, 2048), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, {"kernel": 1}):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(sum(gs)):] == 0).all()
    assert_bf16_parity(o, ref, "bf16 fwd multi-round")


@pytest.mark.parametrize("G", [130, 300])
@pytest.mark.parametrize("placement", [1, 2])
@pytest.mark.parametrize("kernel", [1, 3])
def test_fwd_dx_many_groups(G, placement, kernel):
    """130 groups (a partly filled third chunk of 64 in the prologue's
    register scan) and 300 (past the 256 held in registers: the two-pass
    work-item lookup): the forward and dX against the oracle, with empty
    groups and rows past the total."""
    r = workloads.rng(161, G)
    gs = r.integers(0, 14, G).astype(np.int64)
    gs[::11] = 0
    M = int(gs.sum()) + 29
    wl = workloads.custom(M, 256, 256, gs.tolist(), seed=163 + G, w_std=0.05, with_dy=True)
    total = int(gs.sum())
    cfg = {"kernel": kernel, "placement": placement}
    out = torch.full((M, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, cfg):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    o = to_np64(out)
    assert (o[total:] == 0).all()
    assert_bf16_parity(o, oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes),
                       "fwd G=%d" % G)
    dx = torch.full((M, 256), float("nan"), dtype=torch.bfloat16, device=DEV)
    with tile_config(gmm.OP_DX, cfg):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), _gs(wl), out=dx)
    o = to_np64(dx)
    assert (o[total:] == 0).all()
    assert_bf16_parity(o, oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes),
                       "dx G=%d" % G)
