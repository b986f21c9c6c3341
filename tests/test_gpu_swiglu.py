"""GPU parity of the fused gate+up FP8 GMM ("实现差距：GMM Kernel（V1 vs V2）",
sections 3.5 and 4.2) against the fp64 oracle: the activation within the FP8
tolerance, its 1x128 re-quantisation bit-exact against the oracle's quantiser
applied to the kernel's own fp32 activation (the float decides the code, so
both sides decide from the same value)."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_fp8_parity, sqnr_db, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def fused_problem(M, K, N, gs, seed, x_std=1.0, w_std=0.05, dtype=torch.bfloat16):
    """LHS [M,K] and the [G,K,2N] gate|up weights."""
    wl = workloads.custom(M, K, 2 * N, gs, seed=seed, x_std=x_std, w_std=w_std, dtype=dtype)
    return wl


def run(wl, out_dtype=torch.float32, with_act=False, prequant=False):
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    M, N = wl.M, wl.N // 2
    out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
    aq = asc = None
    if with_act:
        aq = torch.full((M, N), 0x55, dtype=torch.uint8, device=DEV)
        asc = torch.full((M, N // 128), float("nan"), dtype=torch.float32, device=DEV)
    if prequant:
        ql, sl = gmm.gmm_quantize_lhs(wl.x.to(DEV))
        gmm.gmm_fp8_fwd_swiglu(ql, rq, rs, gs, lhs_scale=sl, out=out, act_q=aq, act_scale=asc)
    else:
        gmm.gmm_fp8_fwd_swiglu(wl.x.to(DEV), rq, rs, gs, out=out, act_q=aq, act_scale=asc)
    torch.cuda.synchronize()
    return out, aq, asc


def oracle_act(wl):
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    return oracle.gmm_fp8_swiglu(ql, sl, qr, sr, wl.group_sizes)


def check(wl, out_dtype=torch.float32, with_act=False, prequant=False):
    out, aq, asc = run(wl, out_dtype, with_act, prequant)
    ref = oracle_act(wl)
    o = to_np64(out)
    total = int(wl.group_sizes.sum())
    assert (o[total:] == 0).all(), "rows past the total must be zero"
    assert_fp8_parity(o, ref, "swiglu")
    if with_act:
        q_ref, s_ref = oracle.quantize_lhs(out[:total].float().cpu().numpy())
        assert np.array_equal(aq[:total].cpu().numpy(), q_ref)
        assert np.array_equal(asc[:total].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
        assert (aq[total:].cpu().numpy() == 0).all() and (asc[total:].cpu().numpy() == 0).all()
    return o, ref


@pytest.mark.parametrize("M,K,N,gs", [
    (300, 256, 256, [120, 0, 150, 30]),      # empty group, 300 - 300 = 0 tail
    (1, 128, 256, [1]),                      # one row
    (129, 384, 512, [0, 100]),               # empty first group, 29-row tail
    (1000, 512, 256, [1] * 200 + [700]),     # many size-1 groups, tail of 100
])
def test_shapes_fp32_out_and_requantised(M, K, N, gs):
    check(fused_problem(M, K, N, gs, seed=M + K), torch.float32, with_act=True)


def test_bf16_out():
    check(fused_problem(700, 1024, 512, [300, 0, 350], seed=7), torch.bfloat16)


def test_prequantised_lhs_matches_fused():
    wl = fused_problem(333, 512, 256, [100, 0, 200, 13], seed=9)
    a, _, _ = run(wl, torch.float32, prequant=False)
    b, _, _ = run(wl, torch.float32, prequant=True)
    assert torch.equal(a, b)


def test_agrees_with_unfused_forward():
    """The fused kernel's activation equals silu(P_gate) * P_up of the plain
    forward's fp32 product against the same 2N-column weights (same products,
    same accumulation order; only the exp differs in the last bits)."""
    wl = fused_problem(400, 1024, 256, [130, 0, 200, 70], seed=12)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    p = gmm.gmm_fp8_fwd(wl.x.to(DEV), rq, rs, gs, out_dtype=torch.float32)
    g, u = p[:, :256], p[:, 256:]
    ref = (g / (1.0 + torch.exp(-g)) * u).cpu().numpy().astype(np.float64)
    out, _, _ = run(wl, torch.float32)
    np.testing.assert_allclose(to_np64(out), ref, rtol=1e-5, atol=1e-6)


def test_wi_gate_up_layer():
    """The wi layer with gate and up fused: M=8192, G=32, K=2048, 2 x 512
    columns, top-8 routing; bf16 LHS, activation re-quantised."""
    wl = workloads.make("wi_gate_up", seed=0, with_dy=False)
    o, ref = check(wl, torch.float32, with_act=True)
    print("wi gate+up SQNR vs oracle: %.1f dB" % sqnr_db(ref, o))
