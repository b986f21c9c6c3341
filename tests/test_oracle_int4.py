"""Pins of the oracle's int4-weight path ("实现差距：GMM Kernel（V1 vs V2）",
sections 3.4 and 4.1 name int4 among the sub-byte RHS types; the reading:
codes in [-8, 7], the FP8 path's 128x128 RHS blocks, scale s = a/7 with the
section 3.3 recipe, round half to even).

Independent checks: closed-form blocks whose codes and scale are known,
rounding ties, the error bound and range of any block, exact rational
arithmetic for the scale pair, and the forward against the separately
pinned FP8 oracle (every integer in [-8, 7] is exact in E4M3, so int4
weights are FP8 weights with other codes) and against numpy integer
matmuls on the exact-integer case.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from test_oracle_quant import rn_f32


def block_tensor(vals_128x128: np.ndarray) -> np.ndarray:
    """One expert, one 128x128 block: w [1, 128, 128]."""
    return np.ascontiguousarray(vals_128x128.reshape(1, 128, 128), dtype=np.float32)


@pytest.mark.parametrize("c", [1.0, 0.25, 2.0 ** -20, 2.0 ** 30])
def test_integer_multiples_of_a_power_of_two(c):
    """w = j*c with j in [-7, 7] and some |j| = 7: a = 7c, s = c exactly,
    every code is j."""
    r = np.random.default_rng(1)
    j = r.integers(-7, 8, size=(128, 128))
    j[3, 5] = 7
    q, s = oracle.quantize_rhs_int4(block_tensor(j * c))
    assert s.shape == (1, 1, 1) and s[0, 0, 0] == np.float32(c)
    assert np.array_equal(q[0].astype(np.int64), j)


def test_ties_round_to_even():
    """a = 7 (s = 1, inv = 1): halves round to the even integer."""
    w = np.zeros((128, 128), np.float32)
    vals = [7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 4.5, 6.5, -6.5, 5.5]
    want = [7, 0, 2, 2, 4, 0, -2, -2, 4, 6, -6, 6]
    w[0, :len(vals)] = vals
    q, s = oracle.quantize_rhs_int4(block_tensor(w))
    assert s[0, 0, 0] == 1.0
    assert q[0, 0, :len(vals)].tolist() == want


def test_zero_block_and_independent_blocks():
    w = np.zeros((2, 256, 384), np.float32)
    w[1, 128:, 256:] = np.float32(3.5)          # one non-zero block
    q, s = oracle.quantize_rhs_int4(w)
    assert s.shape == (2, 2, 3)
    nz = np.zeros_like(s, dtype=bool)
    nz[1, 1, 2] = True
    assert (s[~nz] == 0).all() and (q[:, :, :].sum() == 7 * 128 * 128)
    assert s[1, 1, 2] == np.float32(0.5) and (q[1, 128:, 256:] == 7).all()


def test_error_bound_range_and_scale_pair_exactly():
    """Random blocks: s and inv are the correctly rounded a/7 and 1/s (exact
    rationals rounded to fp32 by hand), codes lie in [-7, 7] with +-7 at the
    abs-max, and |w - code*s| <= s/2 up to the rounding of w*inv."""
    r = np.random.default_rng(3)
    w = (r.standard_normal((3, 256, 256)) * r.choice([1e-3, 0.02, 1.0, 300.0], (3, 1, 1))).astype(np.float32)
    q, s = oracle.quantize_rhs_int4(w)
    assert q.min() >= -7 and q.max() <= 7
    for g in range(3):
        for kb in range(2):
            for nb in range(2):
                blk = w[g, 128 * kb:128 * (kb + 1), 128 * nb:128 * (nb + 1)].astype(np.float64)
                cq = q[g, 128 * kb:128 * (kb + 1), 128 * nb:128 * (nb + 1)].astype(np.float64)
                a = np.abs(blk).max()
                sc = rn_f32(Fraction(float(a)) / 7)
                assert s[g, kb, nb] == np.float32(sc)
                inv = rn_f32(1 / Fraction(sc))
                assert np.abs(cq[np.abs(blk) == a]).max() == 7
                err = np.abs(blk - cq * sc)
                assert err.max() <= sc * (0.5 + 8 * 2.0 ** -24) + abs(sc - 1 / inv) * 7


def test_forward_equals_fp8_oracle_on_the_same_integers():
    """int4 codes re-expressed as E4M3 codes (the oracle's encoder, pinned
    against torch's cast) through the pinned FP8 forward give the same
    fp64 result, bit for bit: the int4 forward's indexing, scales and group
    handling match the FP8 forward's."""
    r = np.random.default_rng(5)
    M, K, N, G = 300, 384, 256, 4
    gs = np.array([100, 0, 120, 50], np.int32)
    x = r.standard_normal((M, K)).astype(np.float32)
    w = (r.standard_normal((G, K, N)) * 0.05).astype(np.float32)
    ql, sl = oracle.quantize_lhs(x)
    q4, sr = oracle.quantize_rhs_int4(w)
    q4[2, 7, 9] = -8                             # the one code this quantiser never makes
    q8 = oracle.e4m3_encode(q4.astype(np.float32))
    a = oracle.gmm_fp8_int4(ql, sl, q4, sr, gs)
    b = oracle.gmm_fp8(ql, sl, q8, sr, gs)
    assert np.array_equal(a, b)
    assert (a[gs.sum():] == 0).all()


def test_exact_integer_case_against_numpy():
    """Small-integer LHS values with unit scales (e4m3 codes of integers)
    and int4 codes with unit scales: the forward is an exact integer
    product per group."""
    r = np.random.default_rng(9)
    M, K, N, G = 200, 256, 128, 3
    gs = np.array([70, 0, 110], np.int32)
    xi = r.integers(-8, 9, size=(M, K))
    qi = r.integers(-8, 8, size=(G, K, N)).astype(np.int8)
    ql = oracle.e4m3_encode(xi.astype(np.float32))
    sl = np.ones((M, K // 128), np.float32)
    sr = np.ones((G, K // 128, N // 128), np.float32)
    out = oracle.gmm_fp8_int4(ql, sl, qi, sr, gs)
    off = np.concatenate([[0], np.cumsum(gs)])
    for g in range(G):
        rows = slice(off[g], off[g + 1])
        assert np.array_equal(out[rows], (xi[rows] @ qi[g].astype(np.int64)).astype(np.float64))
    assert (out[off[-1]:] == 0).all()
