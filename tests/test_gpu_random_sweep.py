"""Seeded random sweep of small grouped problems on the GPU against the oracle:
random M, K, N, G, group-size patterns (empty groups, size-1 groups, one
dominant group, rows past the total), LHS dtype (bf16, fp32, or E4M3 codes
with scales) and output dtype, for the FP8-weight, MXFP4-weight and
int4-weight forwards and the fused gate+up SwiGLU forward.  In-kernel codes
and scales bit for bit (in the half of the FP8 cases that ask for them);
outputs within |gpu - ref| <= 1e-3 max(1, rms(ref)) + 1e-2 |ref| and
SQNR > 40 dB (the weights' scale is drawn up to N(0, 1), where outputs are
~20x those of the pages' normalised data, so the absolute term scales with
the output's RMS); rows past the total zero.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_fp8_parity_scaled, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = 24


def group_sizes(r, G, total, pattern):
    if pattern == 0:                                     # uniform routing
        gs = r.multinomial(total, np.full(G, 1.0 / G))
    elif pattern == 1:                                   # one dominant expert
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


def random_problem(seed):
    r = workloads.rng(1000 + seed, 9)
    K = 128 * int(r.integers(1, 9))
    N = 128 * int(r.choice([1, 2, 3, 4, 6, 8]))
    G = int(r.choice([1, 2, 3, 7, 16, 40]))
    total = int(r.integers(1, 900))
    gs = group_sizes(r, G, total, seed % 4)
    M = int(gs.sum()) + int(r.integers(0, 70))           # rows past the total
    dtype = torch.bfloat16 if seed % 3 else torch.float32
    out_dtype = torch.float32 if seed % 2 else torch.bfloat16
    wl = workloads.custom(M, K, N, gs, seed=2000 + seed, w_std=float(r.choice([0.02, 0.05, 1.0])),
                          dtype=dtype)
    return wl, out_dtype


@pytest.mark.parametrize("seed", range(CASES))
def test_fp8_forward_random(seed):
    wl, out_dtype = random_problem(seed)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    # every other case also asks for the in-kernel codes (a kernel variant of
    # its own); the others run the kernels that write only the output
    want_q = seed % 4 < 2
    q = s = None
    if want_q:
        q = torch.zeros((wl.M, wl.K), dtype=torch.uint8, device=DEV)
        s = torch.zeros((wl.M, wl.K // 128), dtype=torch.float32, device=DEV)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    gmm.gmm_fp8_fwd(wl.x.to(DEV), rq, rs, gs, out=out, q_out=q, scale_out=s)
    torch.cuda.synchronize()
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    total = int(wl.group_sizes.sum())
    if want_q:
        assert np.array_equal(q[:total].cpu().numpy(), ql[:total])
        assert np.array_equal(s[:total].cpu().numpy(), sl[:total])
    ref = oracle.gmm_fp8(ql, sl, qr, sr, wl.group_sizes)
    o = to_np64(out)
    assert (o[total:] == 0).all()
    assert_fp8_parity_scaled(o, ref, "random %d (M=%d K=%d N=%d G=%d)" % (seed, wl.M, wl.K, wl.N, wl.G))


@pytest.mark.parametrize("seed", range(CASES))
def test_fp8_forward_prequantised_random(seed):
    """The same problems with the LHS handed in as E4M3 codes and 1x128
    scales (gmm_quantize_lhs output): the kernels that skip the in-kernel
    quantisation, against the same oracle product."""
    wl, out_dtype = random_problem(seed)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    ql_d, sl_d = gmm.gmm_quantize_lhs(wl.x.to(DEV))
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    gmm.gmm_fp8_fwd(ql_d, rq, rs, gs, lhs_scale=sl_d, out=out)
    torch.cuda.synchronize()
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    assert np.array_equal(ql_d.cpu().numpy(), ql) and np.array_equal(sl_d.cpu().numpy(), sl)
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8(ql, sl, qr, sr, wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_fp8_parity_scaled(o, ref, "random prequantised %d (M=%d K=%d N=%d G=%d)" % (seed, wl.M, wl.K, wl.N, wl.G))


@pytest.mark.parametrize("seed", range(CASES))
def test_mxfp4_forward_random(seed):
    wl, out_dtype = random_problem(seed)
    q4, s4 = gmm.gmm_quantize_rhs_mxfp4(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    gmm.gmm_fp8_mxfp4_fwd(wl.x.to(DEV), q4, s4, gs, out=out)
    torch.cuda.synchronize()
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    oq, oe = oracle.quantize_rhs_mxfp4(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8_mxfp4(ql, sl, oq, oe, wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_fp8_parity_scaled(o, ref, "random mxfp4 %d (M=%d K=%d N=%d G=%d)" % (seed, wl.M, wl.K, wl.N, wl.G))


@pytest.mark.parametrize("seed", range(CASES))
def test_int4_forward_random(seed):
    wl, out_dtype = random_problem(seed)
    qi, si = gmm.gmm_quantize_rhs_int4(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    out = torch.full((wl.M, wl.N), float("nan"), dtype=out_dtype, device=DEV)
    gmm.gmm_fp8_int4_fwd(wl.x.to(DEV), qi, si, gs, out=out)
    torch.cuda.synchronize()
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    oq, osr = oracle.quantize_rhs_int4(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8_int4(ql, sl, oq, osr, wl.group_sizes)
    o = to_np64(out)
    assert (o[int(wl.group_sizes.sum()):] == 0).all()
    assert_fp8_parity_scaled(o, ref, "random int4 %d (M=%d K=%d N=%d G=%d)" % (seed, wl.M, wl.K, wl.N, wl.G))


@pytest.mark.parametrize("seed", range(16))
def test_swiglu_forward_random(seed):
    """Fused gate+up ("实现差距：GMM Kernel（V1 vs V2）", sections 3.5 and 4.2):
    N activation columns (a multiple of 256) from [G,K,2N] gate|up weights;
    with fp32 output the 1x128 re-quantisation of the activation too, bit for
    bit against the oracle's quantiser applied to the kernel's fp32 values."""
    r = workloads.rng(5000 + seed, 9)
    K = 128 * int(r.integers(1, 9))
    N = 256 * int(r.integers(1, 4))
    G = int(r.choice([1, 2, 3, 7, 16, 40]))
    gs = group_sizes(r, G, int(r.integers(1, 900)), seed % 4)
    M = int(gs.sum()) + int(r.integers(0, 70))
    dtype = torch.bfloat16 if seed % 3 else torch.float32
    out_dtype = torch.float32 if seed % 2 else torch.bfloat16
    wl = workloads.custom(M, K, 2 * N, gs, seed=6000 + seed, w_std=float(r.choice([0.02, 0.05, 0.5])),
                          dtype=dtype)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    g = torch.from_numpy(gs).to(DEV)
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    with_act = out_dtype == torch.float32
    aq = asc = None
    if with_act:
        aq = torch.full((M, N), 0x55, dtype=torch.uint8, device=DEV)
        asc = torch.full((M, N // 128), float("nan"), dtype=torch.float32, device=DEV)
    gmm.gmm_fp8_fwd_swiglu(wl.x.to(DEV), rq, rs, g, out=out, act_q=aq, act_scale=asc)
    torch.cuda.synchronize()
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8_swiglu(ql, sl, qr, sr, gs)
    o = to_np64(out)
    total = int(gs.sum())
    what = "random swiglu %d (M=%d K=%d N=%d G=%d)" % (seed, M, K, N, G)
    assert (o[total:] == 0).all(), what
    assert_fp8_parity_scaled(o, ref, what)
    if with_act:
        q_ref, s_ref = oracle.quantize_lhs(out[:total].float().cpu().numpy())
        assert np.array_equal(aq[:total].cpu().numpy(), q_ref), what
        assert np.array_equal(asc[:total].cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), what
        assert (aq[total:].cpu().numpy() == 0).all() and (asc[total:].cpu().numpy() == 0).all(), what
