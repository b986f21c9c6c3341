"""GPU parity at the production shape (M=65536, G=256, K=2048, N=512,
top-8 routing with Zipf(1.1)-skewed expert popularity), every output compared
with the fp64 oracle: the FP8 forward in the benchmark's launch configuration
and with its in-kernel codes written out, the MXFP4-weight forward, the bf16
forward, tgmm over all 256 experts and dX over all rows.  Outputs start as NaN,
so an element the kernels never write fails the comparison.

Tolerances: FP8 |gpu - ref| <= 1e-3 + 1e-2 |ref| and SQNR > 40 dB ("GEMM
Kernel 性能优化十问", Q9: kernel vs a CPU reference of the same quantised
computation); bf16 paths 1e-3 + 2e-2 |ref|.  Codes and scales bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, assert_fp8_parity, sqnr_db, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def full():
    wl = workloads.make("full", seed=0, with_dy=True)
    f = {"wl": wl, "x": workloads.as_f32(wl.x), "w": workloads.as_f32(wl.w),
         "dy": workloads.as_f32(wl.dy)}
    f["ql"], f["sl"] = oracle.quantize_lhs(f["x"])
    f["qr"], f["sr"] = oracle.quantize_rhs(f["w"])
    f["fp8_ref"] = oracle.gmm_fp8(f["ql"], f["sl"], f["qr"], f["sr"], wl.group_sizes)
    f["gs"] = torch.from_numpy(wl.group_sizes).to(DEV)
    f["xd"], f["wd"], f["dyd"] = wl.x.to(DEV), wl.w.to(DEV), wl.dy.to(DEV)
    f["total"] = int(wl.group_sizes.sum())
    return f


def nan_out(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def test_fp8_forward_bench_launch_all_rows(full):
    """bf16 LHS quantised in the kernel, bf16 out, no code output: the call
    the benchmark times at this shape."""
    wl = full["wl"]
    rq, rs = gmm.gmm_quantize_rhs(full["wd"])
    out = nan_out((wl.M, wl.N), torch.bfloat16)
    gmm.gmm_fp8_fwd(full["xd"], rq, rs, full["gs"], out=out)
    torch.cuda.synchronize()
    o = to_np64(out)
    assert (o[full["total"]:] == 0).all()
    assert_fp8_parity(o, full["fp8_ref"], "full fp8 forward")
    print("full fp8 forward SQNR vs oracle %.1f dB" % sqnr_db(full["fp8_ref"], o))


def test_fp8_forward_codes_all_rows(full):
    """fp32 out with the in-kernel codes and scales written out: every code
    and scale of every group row bit for bit, every output within the bar."""
    wl = full["wl"]
    rq, rs = gmm.gmm_quantize_rhs(full["wd"])
    out = nan_out((wl.M, wl.N), torch.float32)
    q = torch.zeros((wl.M, wl.K), dtype=torch.uint8, device=DEV)
    s = torch.zeros((wl.M, wl.K // 128), dtype=torch.float32, device=DEV)
    gmm.gmm_fp8_fwd(full["xd"], rq, rs, full["gs"], out=out, q_out=q, scale_out=s)
    torch.cuda.synchronize()
    t = full["total"]
    assert np.array_equal(q[:t].cpu().numpy(), full["ql"][:t])
    assert np.array_equal(s[:t].cpu().numpy().view(np.uint32), full["sl"][:t].view(np.uint32))
    o = to_np64(out)
    assert (o[t:] == 0).all()
    assert_fp8_parity(o, full["fp8_ref"], "full fp8 forward with codes")


def test_mxfp4_forward_all_rows(full):
    wl = full["wl"]
    q4, e8 = gmm.gmm_quantize_rhs_mxfp4(full["wd"])
    out = nan_out((wl.M, wl.N), torch.bfloat16)
    gmm.gmm_fp8_mxfp4_fwd(full["xd"], q4, e8, full["gs"], out=out)
    torch.cuda.synchronize()
    oq4, oe8 = oracle.quantize_rhs_mxfp4(full["w"])
    ref = oracle.gmm_fp8_mxfp4(full["ql"], full["sl"], oq4, oe8, wl.group_sizes)
    o = to_np64(out)
    assert (o[full["total"]:] == 0).all()
    assert_fp8_parity(o, ref, "full mxfp4 forward")


def test_bf16_forward_all_rows(full):
    wl = full["wl"]
    out = nan_out((wl.M, wl.N), torch.bfloat16)
    gmm.gmm_bf16_fwd(full["xd"], full["wd"], full["gs"], out=out)
    torch.cuda.synchronize()
    o = to_np64(out)
    assert (o[full["total"]:] == 0).all()
    assert_bf16_parity(o, oracle.gmm(full["x"], full["w"], wl.group_sizes), "full bf16 forward")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_tgmm_every_expert(full, out_dtype):
    """All 256 experts' dW, with the skewed-routing placement this routing
    takes (tiles spread over the XCDs, groups by size class: every chunk of
    the in-register group scan is reached)."""
    wl = full["wl"]
    dw = nan_out((wl.G, wl.K, wl.N), out_dtype)
    gmm.tgmm_bf16(full["xd"], full["dyd"], full["gs"], out=dw)
    torch.cuda.synchronize()
    ref = oracle.tgmm(full["x"], full["dy"], wl.group_sizes)
    o = to_np64(dw)
    assert not np.isnan(o).any()
    for g in np.flatnonzero(wl.group_sizes == 0):
        assert (o[g] == 0).all()
    assert_bf16_parity(o, ref, "full tgmm")


def test_dx_all_rows(full):
    wl = full["wl"]
    dx = nan_out((wl.M, wl.K), torch.bfloat16)
    gmm.gmm_bf16_dx(full["dyd"], full["wd"], full["gs"], out=dx)
    torch.cuda.synchronize()
    o = to_np64(dx)
    assert (o[full["total"]:] == 0).all()
    assert_bf16_parity(o, oracle.gmm_dx(full["dy"], full["w"], wl.group_sizes), "full dX")
