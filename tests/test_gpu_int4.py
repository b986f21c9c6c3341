"""GPU parity of the int4-weight path against the fp64 oracle.

"实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1 name int4 among the
sub-byte RHS types; the reading (codes in [-8, 7], 128x128 fp32 block scales
s = a/7, round half to even) is the oracle's.  The weight quantiser must
match the oracle's codes and scales bit for bit; the pack call must place
codes made elsewhere, -8 included, exactly where the quantiser does; the
forward is compared like the FP8 forward (|gpu - ref| <= 1e-3 + 1e-2 |ref|
and SQNR > 40 dB), with an exact-integer case compared bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_fp8_parity, pack_int4, sqnr_db, to_np64, unpack_int4

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_quant(w):
    q, s = gmm.gmm_quantize_rhs_int4(w.to(DEV))
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("G,K,N,dtype,std", [
    (3, 256, 128, torch.float32, 0.05),
    (2, 128, 384, torch.bfloat16, 0.02),
    (32, 2048, 512, torch.bfloat16, 0.02),
    (4, 512, 256, torch.float32, 30.0),
])
def test_weight_quantiser_bit_exact(G, K, N, dtype, std):
    r = workloads.rng(G * 11 + K, 3)
    wf = (r.standard_normal((G, K, N)) * std).astype(np.float32)
    wf[0, :128, :128] = 0.0                                   # an all-zero block
    wf[-1, :128, 128 * (N // 128 - 1):] = np.float32(0.25) * r.integers(-7, 8, (128, 128))  # on the grid
    wf[-1, 0, N - 1] = np.float32(7 * 0.25)
    w = workloads.to_bf16(wf) if dtype == torch.bfloat16 else torch.from_numpy(wf)
    q, s = gpu_quant(w)
    oq, os_ = oracle.quantize_rhs_int4(workloads.as_f32(w))
    assert np.array_equal(s.cpu().numpy(), os_)
    assert np.array_equal(unpack_int4(q.cpu().numpy()), oq)


def test_pack_places_codes_like_the_quantiser():
    """Codes made elsewhere, every value of [-8, 7] included, packed by the
    library: the packed bytes equal the documented layout (the test's own
    packer) and, for the quantiser's own codes, the quantiser's output."""
    r = workloads.rng(5, 3)
    codes = r.integers(-8, 8, size=(3, 384, 256)).astype(np.int8)
    codes[0, :16, 0] = np.arange(-8, 8)
    packed = gmm.gmm_pack_rhs_int4(torch.from_numpy(codes).to(DEV)).cpu().numpy()
    assert np.array_equal(packed, pack_int4(codes))
    w = torch.from_numpy((r.standard_normal((2, 256, 512)) * 0.02).astype(np.float32))
    q, _ = gpu_quant(w)
    oq, _ = oracle.quantize_rhs_int4(workloads.as_f32(w))
    again = gmm.gmm_pack_rhs_int4(torch.from_numpy(oq).to(DEV))
    assert torch.equal(again.cpu(), q.cpu())


def run(wl, out_dtype=torch.float32, prequant=False):
    q, s = gpu_quant(wl.w)
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    if prequant:
        ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
        gmm.gmm_fp8_int4_fwd(torch.from_numpy(ql).to(DEV), q, s, gs,
                             lhs_scale=torch.from_numpy(sl).to(DEV), out=out)
    else:
        gmm.gmm_fp8_int4_fwd(wl.x.to(DEV), q, s, gs, out=out)
    torch.cuda.synchronize()
    return to_np64(out)


def reference(wl):
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    q4, sr = oracle.quantize_rhs_int4(workloads.as_f32(wl.w))
    return oracle.gmm_fp8_int4(ql, sl, q4, sr, wl.group_sizes)


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
    check(workloads.custom(M, K, N, gs, seed=M + 3 * N, w_std=0.05, dtype=dtype))


def test_bf16_out_and_prequantised_lhs():
    wl = workloads.custom(333, 512, 512, [100, 0, 200, 13], seed=9)
    check(wl, torch.bfloat16)
    fused = run(wl)
    pre = run(wl, prequant=True)
    assert np.array_equal(fused, pre)        # same codes -> same result bit for bit


@pytest.mark.parametrize("N", [128, 256, 512])
def test_exact_integer_case_bitwise(N):
    """Integer LHS codes with unit scales and int4 codes over all of [-8, 7]
    with unit scales: every partial sum is an integer below 2^24, so the
    fp32 result is exact in any order (all three tile widths)."""
    r = workloads.rng(23 + N, 1)
    M, K, G = 300, 512, 4
    gs = np.array([70, 0, 130, 60], np.int32)
    il = r.integers(-8, 9, size=(M, K))
    ql = oracle.e4m3_encode(il.astype(np.float32))
    sl = np.ones((M, K // 128), np.float32)
    q4 = r.integers(-8, 8, size=(G, K, N)).astype(np.int8)
    sr = np.ones((G, K // 128, N // 128), np.float32)
    packed = gmm.gmm_pack_rhs_int4(torch.from_numpy(q4).to(DEV))
    out = gmm.gmm_fp8_int4_fwd(torch.from_numpy(ql).to(DEV), packed, torch.from_numpy(sr).to(DEV),
                               torch.from_numpy(gs).to(DEV), lhs_scale=torch.from_numpy(sl).to(DEV),
                               out_dtype=torch.float32)
    ref = oracle.gmm_fp8_int4(ql, sl, q4, sr, gs)
    assert np.array_equal(to_np64(out), ref)


def test_empty_group_weights_never_read():
    wl = workloads.custom(200, 256, 256, [90, 0, 110], seed=4)
    q, s = gpu_quant(wl.w)
    q[1] = 0x77                                   # +7 everywhere and a huge scale for the empty expert
    s[1] = 3.0e38
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = gmm.gmm_fp8_int4_fwd(wl.x.to(DEV), q, s, gs, out_dtype=torch.float32)
    o = to_np64(out)
    assert np.isfinite(o).all()
    assert_fp8_parity(o, reference(wl), "poisoned empty group")


@pytest.mark.parametrize("name", ["wi", "wo"])
def test_dev_configs_full(name):
    wl = workloads.make(name, seed=0)
    o, ref = check(wl, torch.bfloat16)
    print("%s int4 SQNR vs oracle: %.1f dB" % (name, sqnr_db(ref, o)))
