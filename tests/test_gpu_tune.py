"""The tile sweep on the GPU: every candidate of a small MXFP4, fused
gate+up and tgmm sweep passes the staged gate against the default
configuration, and a fastest configuration is reported."""
import pytest

from moe_grouped_gemm_gmm_amd import tune

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("phase,shape", [
    ("mxfp4_fwd", (700, 256, 1024, 6)),
    ("swiglu", (600, 256, 256, 4)),
    ("tgmm", (700, 256, 256, 6)),
])
def test_small_sweep(phase, shape):
    t = tune.sweep(phase, shape, steps=20, small_rows=256)
    assert len(t["candidates"]) == len(tune.candidates(phase, shape[2]))
    for r in t["candidates"]:
        assert "error" not in r, r
        assert r["gate_small"] and r["gate_target"], r
        assert r["us"] > 0
    assert t["best"] is not None and t["default_us"] > 0
