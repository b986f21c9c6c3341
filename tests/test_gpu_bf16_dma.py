"""GPU parity of the load-to-LDS bf16 kernel (tile configuration kernel=3:
every accepted pair of depth = LDS stages and residency = workgroups per CU,
so both slice depths, 64 and 32, and the 8-wave 256 x 128 and 128 x 256
tiles) for the
forward, dX and tgmm against the fp64 oracle, at the bf16 bar |gpu - ref| <= 1e-3 + 2e-2 |ref| ("GEMM Kernel
性能优化十问", Q5: the backward is unquantised bf16 with fp32 accumulation):
ragged and empty groups, single rows, groups spanning several 128-row
tiles, tgmm groups whose rows end inside a 64-row slice (rows past the end
zeroed in registers), rows past the total, more than 64 groups, both output
types, both row placements, and the production shape in full."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, tile_config, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    (1, 128, 128, [1]),
    (7, 256, 256, [3, 0, 4]),
    (129, 384, 128, [0, 129]),
    (300, 256, 384, [100, 0, 0, 150]),
    (1000, 512, 256, [1] * 200 + [700]),
    (2000, 256, 128, [600, 0, 3, 1100, 250]),
    (777, 128, 512, [256, 255, 257]),
    (1500, 256, 256, list(np.random.default_rng(3).integers(0, 20, 70))),
]
PAIRS = [(2, 2), (3, 1), (4, 1), (3, 2), (3, 3), (4, 2)]   # (depth, residency)
# every kernel-3 form: the (depth, residency) pairs of 4 waves, and 8 waves
FORMS = [{"depth": d, "residency": r} for d, r in PAIRS] + [{"waves": 8}, {"waves": 8, "tile_n": 256}]
FORM_IDS = ["d%dr%d" % p for p in PAIRS] + ["w8", "w8n256"]


def _fits(form, rows_k, cols):
    """Whether a form's tiles fit: 256 x 128 tgmm tiles need K % 256 == 0
    (rows_k), 128 x 256 tiles the tiled columns % 256 == 0 (cols)."""
    if form.get("tile_n") == 256:
        return cols % 256 == 0
    if form.get("waves") == 8:
        return rows_k is None or rows_k % 256 == 0
    return True


def _gs(wl):
    return torch.from_numpy(wl.group_sizes).to(DEV)


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("placement", [1, 2])
def test_forward(M, K, N, gs, out_dtype, form, placement):
    if not _fits(form, None, N):
        pytest.skip("128 x 256 tiles need N % 256 == 0 (the library rejects this N)")
    wl = workloads.custom(M, K, N, gs, seed=M + K + form.get("depth", 8), w_std=0.05)
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_BF16_FWD, dict(form, kernel=3, placement=placement)):
        gmm.gmm_bf16_fwd(wl.x.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm(workloads.as_f32(wl.x), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "dma fwd")


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("placement", [1, 2])
def test_dx(M, K, N, gs, out_dtype, form, placement):
    if not _fits(form, None, K):
        pytest.skip("128 x 256 tiles need K % 256 == 0 (the library rejects this K)")
    wl = workloads.custom(M, K, N, gs, seed=M + 2 * K + form.get("depth", 8), w_std=0.05, with_dy=True)
    out = torch.full((M, K), float("nan"), dtype=out_dtype, device=DEV)
    with tile_config(gmm.OP_DX, dict(form, kernel=3, placement=placement)):
        gmm.gmm_bf16_dx(wl.dy.to(DEV), wl.w.to(DEV), _gs(wl), out=out)
    ref = oracle.gmm_dx(workloads.as_f32(wl.dy), workloads.as_f32(wl.w), wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_bf16_parity(o, ref, "dma dx")


@pytest.mark.parametrize("M,K,N,gs", CASES)
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
@pytest.mark.parametrize("placement", [0, 1])
def test_tgmm(M, K, N, gs, out_dtype, form, placement):
    if not _fits(form, K, N):
        pytest.skip("this form's tgmm tiles do not divide K x N (the library rejects the shape)")
    wl = workloads.custom(M, K, N, gs, seed=M + 3 * K + form.get("depth", 8), with_dy=True)
    G = len(gs)
    out = torch.full((G, K, N), float("nan"), dtype=out_dtype, device=DEV)
    cfg = dict(form, kernel=3)
    if placement:
        cfg["placement"] = placement
    with tile_config(gmm.OP_TGMM, cfg):
        gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out=out)
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    o = to_np64(out)
    assert not np.isnan(o).any()
    for g in range(G):
        if wl.group_sizes[g] == 0:
            assert (o[g] == 0).all(), "empty group must give exactly zero"
    assert_bf16_parity(o, ref, "dma tgmm")


@pytest.mark.parametrize("form", FORMS, ids=FORM_IDS)
def test_tgmm_slice_tail_reads_nothing_past_the_group(form):
    """Groups of 100 and 150 rows end inside a 64-row slice: the clamped
    loads repeat the group's last row and the kernel zeroes those slots.
    Huge values in the rows past the total, and infinities written into the
    next group's rows of x for a call that only sees group 0's rows, must not
    reach any output."""
    wl = workloads.custom(300, 256, 256, [100, 150], seed=31, with_dy=True)
    x = wl.x.clone()
    x[250:] = 1e30
    with tile_config(gmm.OP_TGMM, dict(form, kernel=3)):
        a = gmm.tgmm_bf16(wl.x.to(DEV), wl.dy.to(DEV), _gs(wl), out_dtype=torch.float32)
        b = gmm.tgmm_bf16(x.to(DEV), wl.dy.to(DEV), _gs(wl), out_dtype=torch.float32)
        x2 = wl.x.clone()
        dy2 = wl.dy.clone()
        x2[100:] = float("inf")
        dy2[100:] = float("inf")
        g0 = torch.tensor([100], dtype=torch.int32, device=DEV)
        c = gmm.tgmm_bf16(x2.to(DEV), dy2.to(DEV), g0, out_dtype=torch.float32)
    assert torch.equal(a, b)
    assert torch.isfinite(c).all()
    assert torch.equal(c[0], a[0])
    ref = oracle.tgmm(workloads.as_f32(wl.x), workloads.as_f32(wl.dy), wl.group_sizes)
    assert_bf16_parity(to_np64(a), ref, "dma tgmm tail")


def test_matches_default_kernel_bitwise_on_exact_integers():
    """Small integers: every partial sum is exact in fp32, so the load-to-LDS
    kernel and the register-fed kernel agree bit for bit (and with the oracle)."""
    rng = np.random.default_rng(5)
    M, K, N, gs = 700, 256, 256, [300, 0, 250, 150]
    x = torch.from_numpy(rng.integers(-3, 4, (M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.integers(-3, 4, (len(gs), K, N)).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(rng.integers(-3, 4, (M, N)).astype(np.float32)).to(torch.bfloat16)
    g = torch.tensor(gs, dtype=torch.int32, device=DEV)
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    ref_f = gmm.gmm_bf16_fwd(xd, wd, g, out_dtype=torch.float32)
    ref_d = gmm.gmm_bf16_dx(dyd, wd, g, out_dtype=torch.float32)
    ref_t = gmm.tgmm_bf16(xd, dyd, g, out_dtype=torch.float32)
    for form in FORMS:
        cfg = dict(form, kernel=3)
        with tile_config(gmm.OP_BF16_FWD, cfg), tile_config(gmm.OP_DX, cfg), tile_config(gmm.OP_TGMM, cfg):
            assert torch.equal(gmm.gmm_bf16_fwd(xd, wd, g, out_dtype=torch.float32), ref_f)
            assert torch.equal(gmm.gmm_bf16_dx(dyd, wd, g, out_dtype=torch.float32), ref_d)
            assert torch.equal(gmm.tgmm_bf16(xd, dyd, g, out_dtype=torch.float32), ref_t)
    exact = oracle.gmm(x.double().numpy(), w.double().numpy(), np.array(gs))
    assert np.array_equal(ref_f.cpu().double().numpy(), exact)


def test_production_shape_full():
    """M=65536, G=256 with the Zipf routing: every row of the forward and dX
    and every tgmm expert, the library's kernel-3 default (3 stages of
    32-deep slices, three workgroups per CU)."""
    wl = workloads.make("full", seed=0, with_dy=True)
    x, dy, w, g = wl.x.to(DEV), wl.dy.to(DEV), wl.w.to(DEV), _gs(wl)
    xs, dys, ws = workloads.as_f32(wl.x), workloads.as_f32(wl.dy), workloads.as_f32(wl.w)
    ref_dx = oracle.gmm_dx(dys, ws, wl.group_sizes)
    ref_dw = oracle.tgmm(xs, dys, wl.group_sizes)
    ref_y = oracle.gmm(xs, ws, wl.group_sizes)
    for cfg in ({"kernel": 3}, {"kernel": 3, "waves": 8}, {"kernel": 3, "waves": 8, "tile_n": 256}):
        with tile_config(gmm.OP_DX, cfg):
            dx = gmm.gmm_bf16_dx(dy, w, g)
        with tile_config(gmm.OP_TGMM, cfg):
            dw = gmm.tgmm_bf16(x, dy, g)
        with tile_config(gmm.OP_BF16_FWD, cfg):
            y = gmm.gmm_bf16_fwd(x, w, g)
        assert_bf16_parity(to_np64(dx), ref_dx, "dma dx full %s" % cfg)
        assert_bf16_parity(to_np64(dw), ref_dw, "dma tgmm full %s" % cfg)
        assert_bf16_parity(to_np64(y), ref_y, "dma fwd full %s" % cfg)
