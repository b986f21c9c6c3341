"""GPU parity: group metadata and the FP8 quantisers, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import unpack_rhs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# ------------------------------------------------------------- metadata -----

@pytest.mark.parametrize("gs,M,tm", [
    ([512], 512, 128),
    ([0, 0, 300, 0], 300, 128),
    ([1, 1, 1, 1], 10, 16),
    ([127, 1, 128, 0, 129], 400, 128),
    ([0, 0, 0], 5, 16),
    ([3, 5, 0, 7], 15, 16),
    ([47, 1, 48, 0, 97], 400, 48),
    ([0, 200, 0, 13], 300, 80),
])
def test_metadata_matches_oracle(gs, M, tm):
    gs = np.array(gs, np.int32)
    ws = gmm.workspace(gmm.OP_METADATA, M, 0, 0, gs.size, DEV)
    off, work, num = gmm.gmm_group_metadata(torch.from_numpy(gs).to(DEV), M, tm, ws=ws)
    ref = oracle.work_list(gs, M, tm)
    n = int(num.item())
    assert n == len(ref)
    assert np.array_equal(work[:n].cpu().numpy(), ref)
    assert np.array_equal(off.cpu().numpy(), oracle.group_offsets(gs, M).astype(np.int32))
    assert gmm.device_status(ws) == 0


def clipped_offsets(gs, M):
    """First row of each group's clipped range, then the clipped total (gmm.h)."""
    o = np.concatenate([[0], np.cumsum(np.maximum(gs.astype(np.int64), 0))])
    return np.minimum(o, M).astype(np.int32)


def expected_status(gs, M):
    return ((gmm.DEV_SUM_GT_M if np.maximum(gs.astype(np.int64), 0).sum() > M else 0)
            | (gmm.DEV_NEGATIVE_SIZE if (gs < 0).any() else 0))


@pytest.mark.parametrize("gs,M,tm", [
    ([128, 128], 128, 128),
    ([100, 100, 100], 250, 64),
    ([5, -3, 7], 20, 16),
    ([-5, 0, 30], 16, 16),
    ([0, 2**31 - 1, 9], 64, 16),       # the metadata kernel writes only its work list
    ([2**31 - 1] * 70, 1000, 48),      # saturation across two chunks of 64 groups
    ([-1] * 65 + [3], 10, 16),
])
def test_metadata_outside_contract(gs, M, tm):
    """Sizes that break the contract: the work list stays inside [0, M) and
    equals the oracle's reading; the status word names what was wrong."""
    gs = np.array(gs, np.int32)
    ws = gmm.workspace(gmm.OP_METADATA, M, 0, 0, gs.size, DEV)
    off, work, num = gmm.gmm_group_metadata(torch.from_numpy(gs).to(DEV), M, tm, ws=ws)
    ref = oracle.work_list(gs, M, tm)
    n = int(num.item())
    assert n == len(ref)
    assert np.array_equal(work[:n].cpu().numpy(), ref)
    assert np.array_equal(off.cpu().numpy(), clipped_offsets(gs, M))
    assert gmm.device_status(ws) == expected_status(gs, M)


def test_metadata_random_and_large_G():
    r = np.random.default_rng(3)
    cases = []
    for _ in range(12):
        G = int(r.integers(1, 300))
        M = int(r.integers(1, 20000))
        tail = int(r.integers(0, min(M, 300)))
        cuts = np.sort(r.integers(0, M - tail + 1, size=G - 1))
        gs = np.diff(np.concatenate([[0], cuts, [M - tail]])).astype(np.int32)
        cases.append((gs, M, int(r.choice([16, 48, 64, 128, 256, 1008]))))
    cases.append((workloads.make("full", with_dy=False).group_sizes, 65536, 128))
    cases.append((workloads.make("full", with_dy=False).group_sizes, 65536, 48))
    for gs, M, tm in cases:
        off, work, num = gmm.gmm_group_metadata(torch.from_numpy(gs).to(DEV), M, tm)
        ref = oracle.work_list(gs, M, tm)
        n = int(num.item())
        assert n == len(ref), (gs.size, M, tm)
        assert np.array_equal(work[:n].cpu().numpy(), ref)


# --------------------------------------------------------- LHS quantiser ----

def _check_lhs(x_cpu: torch.Tensor):
    q, s = gmm.gmm_quantize_lhs(x_cpu.to(DEV))
    rq, rs = oracle.quantize_lhs(workloads.as_f32(x_cpu))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), rq)


@pytest.mark.parametrize("M,K", [(1, 128), (7, 256), (129, 384), (512, 256), (1000, 2048)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_lhs_random(M, K, dtype):
    r = workloads.rng(M * 7 + K, 1)
    x = torch.from_numpy(r.standard_normal((M, K), dtype=np.float32) * np.float32(2.5)).to(dtype)
    _check_lhs(x)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_lhs_edge_blocks(dtype):
    x = torch.zeros((6, 512), dtype=torch.float32)
    x[1, 17] = -3.5                                      # single non-zero
    x[2, :128] = -0.0                                    # negative zeros
    vals = torch.from_numpy(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32))
    x[3, :127] = vals * 8.0                              # power-of-two scale 8
    x[3, 127] = 448.0 * 8.0
    x[4, 128:256] = torch.linspace(-1e-3, 1e-3, 128)
    x[5] = torch.from_numpy(workloads.rng(5, 1).standard_normal(512).astype(np.float32)) * 1e4
    _check_lhs(x.to(dtype))


def test_quantize_lhs_encoder_sweep():
    """Every rounding boundary of the e4m3 grid (and its fp32 neighbours) goes
    through the GPU quantiser with scale exactly 1 (block abs-max 448)."""
    grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((grid[:-1].astype(np.float64) + grid[1:]) / 2).astype(np.float32)
    pts = [grid, mids]
    up, dn = mids.copy(), mids.copy()
    for _ in range(2):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        pts += [up, dn]
    v = np.concatenate(pts)
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 1e-30, -1e-30], np.float32)])
    v = v[np.abs(v) <= 448.0]
    nblk = -(-v.size // 127)
    x = np.zeros((nblk, 128), np.float32)
    x[:, 0] = 448.0                                      # pins s = 1, inv = 1
    flat = x[:, 1:].reshape(-1)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(nblk, 127)
    _check_lhs(torch.from_numpy(x))


# --------------------------------------------------------- RHS quantiser ----

@pytest.mark.parametrize("G,K,N,dtype", [(1, 128, 128, torch.float32), (3, 256, 384, torch.bfloat16),
                                         (4, 256, 256, torch.float32), (2, 2048, 512, torch.bfloat16)])
def test_quantize_rhs(G, K, N, dtype):
    r = workloads.rng(G * 1000 + K + N, 2)
    w = torch.from_numpy(r.standard_normal((G, K, N), dtype=np.float32) * np.float32(0.05)).to(dtype)
    w[0, :128, :128] = 0.0
    q, s = gmm.gmm_quantize_rhs(w.to(DEV))
    rq, rs = oracle.quantize_rhs(workloads.as_f32(w))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(unpack_rhs(q.cpu().numpy()), rq)          # packed MFMA order


def test_quantize_wi_config_bitexact():
    wl = workloads.make("wi", with_dy=False)
    _check_lhs(wl.x)
    q, s = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    rq, rs = oracle.quantize_rhs(workloads.as_f32(wl.w))
    assert np.array_equal(s.cpu().numpy(), rs)
    assert np.array_equal(unpack_rhs(q.cpu().numpy()), rq)
