"""GPU: gmm_fp8_fwd_noalloc, the forward for callers that cannot allocate (its
workspace is the library's static device scratch), called through the C ABI,
gives exactly gmm_fp8_fwd's output on two calls in a row, the second on a
smaller input (the scratch keeps the first call's contents).  Both are also
held to the oracle's FP8 bar."""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_fp8_parity, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def one_call(wl, out_dtype, want_q):
    x = wl.x.to(DEV)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    M, N, K = wl.M, wl.N, wl.K
    outs = []
    for call in (gmm.gmm_fp8_fwd, gmm.gmm_fp8_fwd_noalloc):
        out = torch.full((M, N), float("nan"), dtype=out_dtype, device=DEV)
        q = s = None
        if want_q:
            q = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
            s = torch.zeros((M, K // 128), dtype=torch.float32, device=DEV)
        call(x, rq, rs, gs, out=out, q_out=q, scale_out=s)
        outs.append((out, q, s))
    torch.cuda.synchronize()
    (a, qa, sa), (b, qb, sb) = outs
    assert torch.equal(a, b)
    if want_q:
        assert torch.equal(qa, qb) and torch.equal(sa, sb)
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8(ql, sl, qr, sr, wl.group_sizes)
    assert_fp8_parity(to_np64(b), ref, "noalloc " + wl.name)


def test_noalloc_matches_fp8_fwd_two_calls_second_smaller():
    one_call(workloads.make("wi", seed=0, with_dy=False), torch.bfloat16, want_q=False)
    one_call(workloads.custom(300, 256, 256, [70, 0, 130, 60], seed=41), torch.float32,
             want_q=True)
