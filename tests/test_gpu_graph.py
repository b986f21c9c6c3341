"""The kernels under HIP-graph capture, as the benchmark runs them: one graph
holding the FP8 forward (with the in-kernel codes written out), the LHS
quantiser, the pre-quantised FP8 forward, the MXFP4 and int4 forwards, the
fused gate+up forward (with and without its re-quantised activation) and
the bf16 forward / dX / tgmm is
replayed several times with eager work and synchronisation in between;
every replay must reproduce the eager results bit for bit (the kernels read
group_sizes on the device and clear nothing with memset, so a replay is the
same launch sequence)."""
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_graph_replays_match_eager():
    wl = workloads.custom(700, 512, 512, [200, 0, 300, 77], seed=31, w_std=0.05, with_dy=True)
    x = wl.x.to(DEV)
    w = wl.w.to(DEV)
    dy = wl.dy.to(DEV)
    gs = torch.from_numpy(wl.group_sizes).to(DEV)
    M, K, N, G = wl.M, wl.K, wl.N, wl.G
    rq, rs = gmm.gmm_quantize_rhs(w)
    q4, s4 = gmm.gmm_quantize_rhs_mxfp4(w)
    qi, si = gmm.gmm_quantize_rhs_int4(w)
    ql, sl = gmm.gmm_quantize_lhs(x)
    gq, gsc = gmm.gmm_quantize_rhs(torch.cat([w, w.flip(1)], dim=2).contiguous())
    outs = {
        "fp8": torch.zeros((M, N), dtype=torch.bfloat16, device=DEV),
        "q": torch.zeros((M, K), dtype=torch.uint8, device=DEV),
        "s": torch.zeros((M, K // 128), dtype=torch.float32, device=DEV),
        "mx": torch.zeros((M, N), dtype=torch.float32, device=DEV),
        "pre": torch.zeros((M, N), dtype=torch.bfloat16, device=DEV),
        "i4": torch.zeros((M, N), dtype=torch.bfloat16, device=DEV),
        "act": torch.zeros((M, N), dtype=torch.bfloat16, device=DEV),
        "act32": torch.zeros((M, N), dtype=torch.float32, device=DEV),
        "aq": torch.zeros((M, N), dtype=torch.uint8, device=DEV),
        "as": torch.zeros((M, N // 128), dtype=torch.float32, device=DEV),
        "bf": torch.zeros((M, N), dtype=torch.bfloat16, device=DEV),
        "dx": torch.zeros((M, K), dtype=torch.bfloat16, device=DEV),
        "dw": torch.zeros((G, K, N), dtype=torch.float32, device=DEV),
    }
    total = int(wl.group_sizes.sum())
    # the in-kernel codes and scales are defined for the rows of the groups
    rows = {"q": total, "s": total}
    made = {}   # the quantiser's outputs, allocated by the call (in the graph's pool when captured)

    def run():
        gmm.gmm_fp8_fwd(x, rq, rs, gs, out=outs["fp8"], q_out=outs["q"], scale_out=outs["s"])
        made["ql"], made["sl"] = gmm.gmm_quantize_lhs(x)
        gmm.gmm_fp8_fwd(ql, rq, rs, gs, lhs_scale=sl, out=outs["pre"])
        gmm.gmm_fp8_mxfp4_fwd(x, q4, s4, gs, out=outs["mx"])
        gmm.gmm_fp8_int4_fwd(x, qi, si, gs, out=outs["i4"])
        gmm.gmm_fp8_fwd_swiglu(x, gq, gsc, gs, out=outs["act"])
        gmm.gmm_fp8_fwd_swiglu(x, gq, gsc, gs, out=outs["act32"], act_q=outs["aq"], act_scale=outs["as"])
        gmm.gmm_bf16_fwd(x, w, gs, out=outs["bf"])
        gmm.gmm_bf16_dx(dy, w, gs, out=outs["dx"])
        gmm.tgmm_bf16(x, dy, gs, out=outs["dw"])

    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    eager.update({k: v.clone() for k, v in made.items()})

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        run()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in list(outs.values()) + list(made.values()):
            v.zero_()                                   # eager work between replays
        junk = (torch.randn(1 << 20, device=DEV) * 3).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for k, v in list(outs.items()) + list(made.items()):
            n = rows.get(k, v.shape[0])
            assert torch.equal(v[:n], eager[k][:n]), "replay %d: %s differs from the eager result" % (rep, k)
