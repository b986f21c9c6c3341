"""Pins of the oracle's fused gate+up activation ("实现差距：GMM Kernel（V1 vs
V2）", sections 3.5 and 4.2: gate columns first, then up; the result is
silu(gate) * up)."""
import math

import numpy as np
import scipy.special

import oracle
import workloads


def test_matches_library_logistic():
    r = np.random.default_rng(0)
    g = r.standard_normal((37, 64)) * 4.0
    u = r.standard_normal((37, 64)) * 2.0
    out = oracle.swiglu(np.concatenate([g, u], axis=1))
    ref = g * scipy.special.expit(g) * u
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-300)


def test_closed_forms():
    ln3 = math.log(3.0)
    z = np.array([[0.0, ln3, -ln3, 40.0, -40.0]])
    out = oracle.swiglu(np.concatenate([z, np.ones_like(z)], axis=1))[0]
    assert out[0] == 0.0                                  # silu(0) = 0
    assert abs(out[1] - 0.75 * ln3) < 1e-15               # sigmoid(ln 3) = 3/4
    assert abs(out[1] - out[2] - ln3) < 1e-15             # silu(z) - silu(-z) = z
    assert abs(out[3] - 40.0) < 1e-12 and abs(out[4]) < 1e-15


def test_gate_is_first_half_up_second():
    g = np.array([[2.0, -1.0]])
    u = np.array([[3.0, 5.0]])
    a = oracle.swiglu(np.concatenate([g, u], axis=1))
    b = oracle.swiglu(np.concatenate([u, g], axis=1))
    np.testing.assert_allclose(a, g / (1 + np.exp(-g)) * u, rtol=1e-15)
    assert not np.allclose(a, b)


def test_fused_weights_equal_separate_projections():
    """Quantising the [G,K,2N] concatenation with 128x128 blocks is quantising
    the gate and up weights separately, so the fused product is the pair of
    separate products side by side (bitwise), and the activation follows."""
    wl = workloads.custom(300, 256, 256, [120, 0, 150, 30], seed=3, w_std=0.05)
    r = workloads.rng(3, 2)
    wu = (r.standard_normal(workloads.as_f32(wl.w).shape) * 0.05).astype(np.float32)
    wg = workloads.as_f32(wl.w)
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qc, sc = oracle.quantize_rhs(np.concatenate([wg, wu], axis=2))
    qg, sg = oracle.quantize_rhs(wg)
    qu, su = oracle.quantize_rhs(wu)
    fused = oracle.gmm_fp8(ql, sl, qc, sc, wl.group_sizes)
    pg = oracle.gmm_fp8(ql, sl, qg, sg, wl.group_sizes)
    pu = oracle.gmm_fp8(ql, sl, qu, su, wl.group_sizes)
    assert np.array_equal(fused, np.concatenate([pg, pu], axis=1))
    act = oracle.gmm_fp8_swiglu(ql, sl, qc, sc, wl.group_sizes)
    np.testing.assert_allclose(act, pg / (1 + np.exp(-pg)) * pu, rtol=1e-14, atol=1e-300)
    total = int(wl.group_sizes.sum())
    assert (act[total:] == 0).all()
