"""The tile-sweep harness's host logic (no GPU): candidate enumeration, the
tolerance gate, staged gating and best-configuration choice with a fake
runner standing in for the child processes."""
import json

import numpy as np
import pytest

from moe_grouped_gemm_gmm_amd import tune


def test_candidates_per_phase():
    c = tune.candidates("fp8_fwd", 512)
    assert c[0] == {}
    assert len(c) == 1 + 2 + 6
    ws = [e for e in c if e.get("GMM_FP8_WS") == "1"]
    assert {e["GMM_FP8_WS_WAVES"] for e in ws} == {"8", "16"}
    assert all(e["GMM_FP8_WN"] == "64" and e["GMM_FP8_TM"] == "48" for e in ws)
    c256 = tune.candidates("fp8_fwd_prequant", 256)
    assert not any(e.get("GMM_FP8_WS") == "1" for e in c256)
    assert {e["GMM_FP8_WN"] for e in c256[1:]} == {"32", "16"}
    assert [e.get("GMM_MXFP4_TN") for e in tune.candidates("mxfp4_fwd", 384)] == [None, "128"]
    assert [e.get("GMM_MXFP4_TN") for e in tune.candidates("mxfp4_fwd", 1024)] == [None, "512", "256", "128"]
    assert [e.get("GMM_SWIGLU_TM") for e in tune.candidates("swiglu", 512)] == [None, "48", "64"]
    for phase in ("bf16_fwd", "tgmm", "dx"):
        assert [e.get("GMM_BF16_MINB") for e in tune.candidates(phase, 512)] == [None, "2", "3"]
    names = [tune.env_name(e) for e in tune.candidates("fp8_fwd", 512)]
    assert len(set(names)) == len(names) and names[0] == "default"
    with pytest.raises(ValueError):
        tune.candidates("nope", 512)


def test_gate_excess():
    ref = np.array([[1.0, -2.0, 0.0]])
    assert tune.gate_excess(ref.copy(), ref) < 0
    ok = ref + np.array([[0.01, -0.02, 0.001]])        # at the tolerance edge: 1e-3 + 1e-2|ref|
    assert tune.gate_excess(ok, ref) <= 1e-12
    bad = ref + np.array([[0.0, 0.0, 0.01]])
    assert tune.gate_excess(bad, ref) == pytest.approx(0.009)
    assert tune.gate_excess(np.array([[1.0, np.nan, 0.0]]), ref) == float("inf")
    assert tune.gate_excess(np.zeros((2, 3)), ref) == float("inf")


class FakeRunner:
    """Writes a deterministic output per (shape, config) and reports a time;
    one configuration is wrong on the small problem, one only on the target,
    one crashes."""

    def __init__(self):
        self.calls = []

    def __call__(self, phase, shape, env, seed, steps, save):
        self.calls.append((tuple(shape), tune.env_name(env), steps))
        M, K, N, G = shape
        out = np.arange(M * N, dtype=np.float32).reshape(M, N) / (M * N)
        name = tune.env_name(env)
        if name == "GMM_MXFP4_TN=256":
            out = out + 0.5                                  # wrong everywhere
        if name == "GMM_MXFP4_TN=128" and M > 512:
            out = out * 1.1                                  # wrong only at the target
        if name == "GMM_MXFP4_TN=512" and M > 512:
            return {"error": "boom"}
        np.save(save, out)
        us = {"default": 10.0, "GMM_MXFP4_TN=512": 5.0, "GMM_MXFP4_TN=256": 1.0,
              "GMM_MXFP4_TN=128": 2.0}[name]
        return {"us": us} if steps else {}


def test_sweep_stages_and_best():
    fr = FakeRunner()
    t = tune.sweep("mxfp4_fwd", (2048, 256, 1024, 8), steps=10, runner=fr)
    rows = {r["config"]: r for r in t["candidates"]}
    assert rows["default"]["gate_target"] and rows["default"]["us"] == 10.0
    assert rows["GMM_MXFP4_TN=256"]["gate_small"] is False and "gate_target" not in rows["GMM_MXFP4_TN=256"]
    assert rows["GMM_MXFP4_TN=128"]["gate_small"] and rows["GMM_MXFP4_TN=128"]["gate_target"] is False
    assert rows["GMM_MXFP4_TN=512"]["error"] == "boom"
    assert t["best"]["config"] == "default" and t["default_us"] == 10.0
    assert t["small_shape"] == [512, 256, 1024, 4]
    # the failing-on-small candidate never ran at the target size
    assert not any(c[1] == "GMM_MXFP4_TN=256" and c[0][0] == 2048 for c in fr.calls)
    # only target-size runs are timed
    assert all(shape[0] == 2048 for shape, name, steps in fr.calls if steps)
    assert any(steps for shape, name, steps in fr.calls)
    json.dumps(t)                                           # serialisable


def test_default_failure_raises():
    def runner(phase, shape, env, seed, steps, save):
        return {"error": "no gpu"}
    with pytest.raises(RuntimeError):
        tune.sweep("swiglu", (600, 256, 512, 4), runner=runner)
