"""GPU parity of the MXFP4-weight path against the fp64 oracle.

"实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1 (sub-byte RHS, MXFP4
first); format and conversion from the OCP MX specification v1.0.  The
weight quantiser must match the oracle's codes and E8M0 scales bit for bit;
the forward is compared like the FP8 forward (only the fp32 accumulation
order and the output rounding differ): |gpu - ref| <= 1e-3 + 1e-2 |ref| and
SQNR > 40 dB, with an exact-integer case compared bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_fp8_parity, pack_mxfp4, sqnr_db, to_np64, unpack_mxfp4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_quant(w):
    q, s = gmm.gmm_quantize_rhs_mxfp4(w.to(DEV))
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("G,K,N,dtype,std", [
    (3, 256, 128, torch.float32, 0.05),
    (2, 128, 384, torch.bfloat16, 0.02),
    (32, 2048, 512, torch.bfloat16, 0.02),
    (4, 512, 256, torch.float32, 30.0),
])
def test_weight_quantiser_bit_exact(G, K, N, dtype, std):
    r = workloads.rng(G * 7 + K, 3)
    wf = (r.standard_normal((G, K, N)) * std).astype(np.float32)
    wf[0, :32, 5] = 0.0                                   # an all-zero block
    wf[-1, 64:96, 3] = -0.0
    wf[0, 32:64, 7] = np.float32(6.0 * 2.0 ** -3)         # exactly on the grid
    w = workloads.to_bf16(wf) if dtype == torch.bfloat16 else torch.from_numpy(wf)
    q, s = gpu_quant(w)
    codes, e8 = unpack_mxfp4(q.cpu().numpy(), s.cpu().numpy())
    oq, oe = oracle.quantize_rhs_mxfp4(workloads.as_f32(w))
    assert np.array_equal(e8, oe)
    assert np.array_equal(codes, oq)


def run(wl, out_dtype=torch.float32, prequant=False):
    q, s = gpu_quant(wl.w)
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    if prequant:
        ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
        gmm.gmm_fp8_mxfp4_fwd(torch.from_numpy(ql).to(DEV), q, s, gs,
                              lhs_scale=torch.from_numpy(sl).to(DEV), out=out)
    else:
        gmm.gmm_fp8_mxfp4_fwd(wl.x.to(DEV), q, s, gs, out=out)
    torch.cuda.synchronize()
    return to_np64(out)


def reference(wl):
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    q4, e8 = oracle.quantize_rhs_mxfp4(workloads.as_f32(wl.w))
    return oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, wl.group_sizes)


def check(wl, out_dtype=torch.float32, prequant=False):
    o = run(wl, out_dtype, prequant)
    ref = reference(wl)
    total = int(wl.group_sizes.sum())
    assert (o[total:] == 0).all(), "rows past the total must be zero"
    assert_fp8_parity(o, ref, wl.name)
    return o, ref


@pytest.mark.parametrize("M,K,N,gs", [
    (1, 128, 128, [1]),
    (7, 256, 256, [3, 0, 4]),
    (129, 384, 128, [0, 129]),
    (300, 256, 384, [100, 0, 0, 150]),
    (1000, 512, 256, [1] * 200 + [800]),
    (640, 256, 512, [128, 128, 128, 128, 128]),
    (513, 128, 1024, [0, 0, 513, 0]),
])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_edge_shapes(M, K, N, gs, dtype):
    """N = 128, 256, 384 and 512, 1024 run the 128-, 256- and 512-column tiles."""
    check(workloads.custom(M, K, N, gs, seed=M + N, w_std=0.05, dtype=dtype))


def test_bf16_out_and_prequantised_lhs():
    wl = workloads.custom(333, 512, 512, [100, 0, 200, 13], seed=9)
    check(wl, torch.bfloat16)
    fused = run(wl)
    pre = run(wl, prequant=True)
    assert np.array_equal(fused, pre)        # same codes -> same result bit for bit


def test_exact_integer_case_bitwise():
    """Integer LHS codes with unit scales, E2M1 codes and E8M0 exponents 126..129:
    every partial sum is a multiple of 1/2 below 2^23, so the fp32 result is
    exact in any order."""
    r = workloads.rng(21, 1)
    M, K, N, G = 300, 512, 256, 4
    gs = np.array([70, 0, 130, 60], np.int32)
    il = r.integers(-8, 9, size=(M, K))
    ql = oracle.e4m3_encode(il.astype(np.float32))
    sl = np.ones((M, K // 128), np.float32)
    vals = r.choice(np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -2, -3, -6]), size=(G, K, N))
    q4 = oracle.e2m1_encode(vals)
    e8 = r.integers(126, 130, size=(G, K // 32, N)).astype(np.uint8)
    qp, sp = pack_mxfp4(q4, e8)
    out = gmm.gmm_fp8_mxfp4_fwd(torch.from_numpy(ql).to(DEV), torch.from_numpy(qp).to(DEV),
                                torch.from_numpy(sp).to(DEV), torch.from_numpy(gs).to(DEV),
                                lhs_scale=torch.from_numpy(sl).to(DEV), out_dtype=torch.float32)
    ref = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, gs)
    assert np.array_equal(to_np64(out), ref)


def test_empty_group_weights_never_read():
    wl = workloads.custom(200, 256, 256, [90, 0, 110], seed=4)
    q, s = gpu_quant(wl.w)
    q[1] = 0x77                                   # +-6 everywhere and scale 2^127 for the empty expert
    s[1] = 254
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = gmm.gmm_fp8_mxfp4_fwd(wl.x.to(DEV), q, s, gs, out_dtype=torch.float32)
    o = to_np64(out)
    assert np.isfinite(o).all()
    assert_fp8_parity(o, reference(wl), "poisoned empty group")


@pytest.mark.parametrize("name", ["wi", "wo"])
def test_dev_configs_full(name):
    wl = workloads.make(name, seed=0)
    o, ref = check(wl, torch.bfloat16)
    print("%s MXFP4 SQNR vs oracle: %.1f dB" % (name, sqnr_db(ref, o)))
