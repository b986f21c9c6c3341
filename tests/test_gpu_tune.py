"""The tile search on the GPU.

Every configuration the search can pick, of every phase, is checked against
the CPU oracle ("GEMM Kernel 性能优化十问", Q9.3, first layer: a single grouped
call compared with the CPU reference over the shape combinations and all
tiling configurations) at a small ragged shape (an empty group, rows past
the total) and at the wi/wo development shapes; then a staged search (Q9.4)
runs with the oracle as its reference."""
import numpy as np
import pytest

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, assert_fp8_parity
from moe_grouped_gemm_gmm_amd import tune

pytestmark = pytest.mark.gpu


def oracle_reference(p: tune.Problem) -> np.ndarray:
    """The phase's result from the fp64 oracle on the problem's own inputs."""
    x = workloads.as_f32(p.x)
    w = workloads.as_f32(p.w)
    gs = p.gs_host
    if p.phase in ("bf16_fwd", "tgmm", "dx"):
        dy = workloads.as_f32(p.dy)
        if p.phase == "bf16_fwd":
            return oracle.gmm(x, w, gs)
        if p.phase == "tgmm":
            return oracle.tgmm(x, dy, gs)
        return oracle.gmm_dx(dy, w, gs)
    ql, sl = oracle.quantize_lhs(x)
    if p.phase == "mxfp4_fwd":
        q4, e8 = oracle.quantize_rhs_mxfp4(w)
        return oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, gs)
    if p.phase == "int4_fwd":
        qi, si = oracle.quantize_rhs_int4(w)
        return oracle.gmm_fp8_int4(ql, sl, qi, si, gs)
    qr, sr = oracle.quantize_rhs(w)
    if p.phase == "swiglu":
        return oracle.gmm_fp8_swiglu(ql, sl, qr, sr, gs)
    return oracle.gmm_fp8(ql, sl, qr, sr, gs)


CASES = [
    ("fp8_fwd", (700, 512, 1024, 6)), ("fp8_fwd", (8192, 2048, 512, 32)),
    ("fp8_fwd", (8192, 512, 2048, 32)),
    ("fp8_fwd_prequant", (700, 512, 1024, 6)), ("fp8_fwd_prequant", (8192, 2048, 512, 32)),
    ("mxfp4_fwd", (700, 512, 1024, 6)), ("mxfp4_fwd", (8192, 2048, 512, 32)),
    ("int4_fwd", (700, 512, 1024, 6)), ("int4_fwd", (8192, 2048, 512, 32)),
    ("swiglu", (700, 512, 512, 6)), ("swiglu", (8192, 2048, 512, 32)),
    ("bf16_fwd", (900, 256, 512, 6)), ("dx", (900, 256, 512, 6)), ("tgmm", (900, 256, 512, 6)),
    ("tgmm", (8192, 2048, 512, 32)),
]


@pytest.mark.parametrize("phase,shape", CASES)
def test_every_configuration_matches_oracle(phase, shape):
    cands = tune.candidates(phase, shape)
    assert len(cands) >= 2
    routing = "zipf" if phase == "tgmm" else "uniform"
    gs = tune.group_sizes(shape[0], shape[3], 3, routing)
    if shape[0] < 8192:                       # an empty group and rows past the total
        gs[0] += gs[1]
        gs[1] = 0
        gs[-1] = max(0, gs[-1] - 37)
    p = tune.Problem(phase, shape, seed=3, routing=routing, sizes=gs)
    ref = oracle_reference(p)
    op = tune.op_of(phase)
    try:
        for cfg in cands:
            gmm.set_tile_config(op, cfg or None)
            out = p.run()
            what = "%s %s %s" % (phase, shape, tune.config_name(cfg))
            if phase in ("bf16_fwd", "tgmm", "dx"):
                assert_bf16_parity(out, ref, what)
            else:
                assert_fp8_parity(out, ref, what)
    finally:
        gmm.set_tile_config(op, None)


@pytest.mark.parametrize("phase,shape", [("fp8_fwd", (2000, 1024, 512, 8)),
                                         ("tgmm", (2000, 256, 512, 8))])
def test_staged_search_with_oracle_reference(phase, shape):
    t = tune.search(phase, shape, steps=10, small_rows=256, reference=oracle_reference)
    rows = t["candidates"]
    assert len(rows) == len(tune.candidates(phase, shape))
    for r in rows:
        assert r["screen"]["pass"], r
        assert r["explore"]["pass"] and r["us"] > 0, r
    verified = [r for r in rows if "verify" in r]
    assert 1 <= len(verified) <= tune.VERIFY_TOP
    assert t["best"] is not None and t["best"]["verify"]["pass"]
    assert t["best"]["us"] == min(r["us"] for r in verified if r["verify"]["pass"])
