"""Pins of the oracle's blockwise quantisers (LHS 1x128, RHS 128x128).

Recipe ("实现差距：GMM Kernel（V1 vs V2）", section 3.3, with the block shapes
of "GEMM Kernel 性能优化十问", Q2): a = abs-max of the block, s = a/448,
inv = 0 if s == 0 else 1/s, code = e4m3(x*inv), each step one correctly
rounded fp32 operation.

Independent checks: the same recipe in numpy fp32 arithmetic with torch's
e4m3 cast; exact rational arithmetic (fractions) with round-to-nearest-even
to fp32 written out here; closed forms.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def numpy_recipe_blocks(blocks: np.ndarray):
    """blocks: [nblk, n] fp32 -> (codes [nblk,n], scales [nblk]) in numpy fp32."""
    a = np.max(np.abs(blocks), axis=1).astype(np.float32)
    s = (a / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(s == 0, np.float32(0.0), np.float32(1.0) / s).astype(np.float32)
    y = (blocks * inv[:, None]).astype(np.float32)
    return torch_e4m3(y), s


def rn_f32(q: Fraction) -> float:
    """Round a rational to the nearest fp32 value, ties to even (normal and subnormal)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    q = abs(q)
    e = math.floor(math.log2(q.numerator) - math.log2(q.denominator))
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    t = q / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n * quantum)


def test_lhs_matches_numpy_recipe_random():
    r = np.random.default_rng(7)
    x = r.standard_normal((257, 512), dtype=np.float32) * np.float32(3.0)
    x[5, :128] = 0.0                       # zero block
    x[6, 128:256] = -0.0                   # negative-zero block
    x[7, 256:384] *= np.float32(1e-20)     # tiny but in-contract block
    x[8, 384:] *= np.float32(1e20)
    q, s = oracle.quantize_lhs(x)
    cq, cs = numpy_recipe_blocks(x.reshape(-1, 128))
    assert np.array_equal(s.reshape(-1).view(np.uint32), cs.view(np.uint32))
    assert np.array_equal(q.reshape(-1, 128), cq)


def test_lhs_bf16_inputs_match_numpy_recipe():
    r = np.random.default_rng(8)
    xb = torch.from_numpy(r.standard_normal((64, 2048), dtype=np.float32)).to(torch.bfloat16)
    x = xb.float().numpy()
    q, s = oracle.quantize_lhs(x)
    cq, cs = numpy_recipe_blocks(x.reshape(-1, 128))
    assert np.array_equal(s.reshape(-1), cs)
    assert np.array_equal(q.reshape(-1, 128), cq)


def test_lhs_scale_and_codes_exact_rational():
    r = np.random.default_rng(9)
    x = r.standard_normal((6, 128), dtype=np.float32) * np.float32(0.37)
    q, s = oracle.quantize_lhs(x)
    for m in range(x.shape[0]):
        a = max(abs(Fraction(float(v))) for v in x[m])
        s_ref = rn_f32(a / 448)
        assert float(s[m, 0]) == s_ref
        inv = rn_f32(1 / Fraction(s_ref))
        y = np.array([rn_f32(Fraction(float(v)) * Fraction(inv)) for v in x[m]], np.float32)
        assert np.array_equal(q[m], torch_e4m3(y))


def test_lhs_closed_forms():
    x = np.zeros((4, 256), np.float32)
    x[1, 17] = -3.5                        # single non-zero value in block 0
    x[2, :128] = -0.0                      # all negative zeros
    j = 3                                  # power-of-two scale: a = 448 * 2^j
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    x[3, :127] = vals * np.float32(2.0 ** j)
    x[3, 127] = 448.0 * 2.0 ** j
    x[3, 128:] = -x[3, :128]
    q, s = oracle.quantize_lhs(x)
    assert s[0].tolist() == [0.0, 0.0] and not q[0].any()
    assert s[1, 0] == np.float32(3.5) / np.float32(448.0) and s[1, 1] == 0.0
    assert q[1, 17] == 0xFE and np.count_nonzero(q[1]) == 1
    assert (q[2, :128] == 0x80).all() and s[2, 0] == 0.0
    assert s[3].tolist() == [2.0 ** j, 2.0 ** j]
    assert q[3, :127].tolist() == list(range(0x7F))     # each value maps to its own code
    assert q[3, 127] == 0x7E
    assert q[3, 128:255].tolist() == [c | 0x80 for c in range(0x7F)]


def test_rhs_matches_numpy_recipe():
    r = np.random.default_rng(10)
    G, K, N = 3, 256, 384
    w = r.standard_normal((G, K, N), dtype=np.float32) * np.float32(0.05)
    w[1, 128:, :128] = 0.0
    q, s = oracle.quantize_rhs(w)
    blocks = w.reshape(G, K // 128, 128, N // 128, 128).transpose(0, 1, 3, 2, 4).reshape(-1, 128 * 128)
    cq, cs = numpy_recipe_blocks(blocks)
    assert np.array_equal(s.reshape(-1), cs)
    qb = q.reshape(G, K // 128, 128, N // 128, 128).transpose(0, 1, 3, 2, 4).reshape(-1, 128 * 128)
    assert np.array_equal(qb, cq)
    assert s[1, 1, 0] == 0.0


def test_rhs_power_of_two_block():
    w = np.zeros((1, 128, 128), np.float32)
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    w[0, 0, :127] = vals * np.float32(0.25)
    w[0, 5, 9] = 448.0 * 0.25
    q, s = oracle.quantize_rhs(w)
    assert s[0, 0, 0] == 0.25
    assert q[0, 0, :127].tolist() == list(range(0x7F))
    assert q[0, 5, 9] == 0x7E


# ------------------------------------------------------- the scale pair ----

def contract_amax_sample(seed=0, per_exp=64):
    """Block abs-maxima across the contract's range [2^-100, FLT_MAX]: for each
    exponent, the binade's first and last significands and random ones."""
    r = np.random.default_rng(seed)
    bits = []
    for e in range(-100, 128):
        base = (e + 127) << 23
        sig = np.concatenate([[0, 1, (1 << 23) - 1], r.integers(0, 1 << 23, size=per_exp)])
        bits.append(base + sig)
    return np.concatenate(bits).astype(np.uint32).view(np.float32)


def test_quant_scales_exact_rational():
    """s = RN(a/448) and inv = RN(1/s), against exact rational arithmetic."""
    a = contract_amax_sample(per_exp=6)
    s, inv = oracle.quant_scales(a)
    for ai, si, ii in zip(a.tolist(), s.tolist(), inv.tolist()):
        want_s = rn_f32(Fraction(ai) / 448)
        assert si == want_s, (ai, si, want_s)
        assert ii == rn_f32(1 / Fraction(want_s)), (ai, ii)


def test_quant_scales_binade_vs_numpy_division():
    """Every significand of one binade of a (the recipe's scaling by 2^k only
    moves the exponent inside the contract's range), against numpy's IEEE fp32
    division."""
    a = ((np.uint32(136) << 23) + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)
    s, inv = oracle.quant_scales(a)
    ns = a / np.float32(448.0)
    assert np.array_equal(s.view(np.uint32), ns.view(np.uint32))
    assert np.array_equal(inv.view(np.uint32), (np.float32(1.0) / ns).view(np.uint32))


def test_quant_scales_closed_forms():
    a = np.array([0.0, 448.0, 448.0 * 2 ** -90, 448.0 * 2 ** 100, 224.0], np.float32)
    s, inv = oracle.quant_scales(a)
    assert s.tolist() == [0.0, 1.0, 2.0 ** -90, 2.0 ** 100, 0.5]
    assert inv.tolist() == [0.0, 1.0, 2.0 ** 90, 2.0 ** -100, 2.0]
