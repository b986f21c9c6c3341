"""Pins of the oracle's MXFP4 weight path.

Sources: "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1 (sub-byte RHS
types, MXFP4 first), and the OCP Microscaling (MX) specification v1.0 for the
format: 32 E2M1 elements share one E8M0 power-of-two scale, the shared
exponent of a block is floor(log2(max|v|)) minus 2 (the largest E2M1
exponent), elements are rounded to E2M1 and clamped to +-6.  The LHS keeps
the FP8 1x128 recipe.  Every pin below checks the oracle against a closed
form, a defining property over a dense sweep, exact integer arithmetic, or
the already pinned FP8 oracle.
"""
import numpy as np
import pytest

import oracle
import workloads

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e2m1_decode_closed_form():
    # code = sign | exponent(2) | mantissa(1); exponent 0 is subnormal (0, 0.5)
    vals = oracle.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == list(GRID)
    assert list(vals[8:]) == list(-GRID)


def test_e2m1_encode_round_trip_and_signs():
    codes = np.arange(16, dtype=np.uint8)
    vals = oracle.e2m1_decode(codes)
    back = oracle.e2m1_encode(vals)
    assert np.array_equal(back[1:], codes[1:])
    assert back[0] == 0 and back[8] == 8           # +0 and -0 keep their sign
    assert oracle.e2m1_encode([-1e-9])[0] == 8


def test_e2m1_encode_is_nearest_with_even_ties():
    """Dense sweep: the decoded value is a nearest grid point; at the exact
    midpoints the code with mantissa bit 0 wins; |y| >= 6 saturates."""
    y = np.concatenate([np.linspace(0, 7.5, 6001), (GRID[1:] + GRID[:-1]) / 2])
    codes = oracle.e2m1_encode(y)
    dec = oracle.e2m1_decode(codes)
    dist = np.abs(y[:, None] - GRID[None, :]).min(axis=1)
    assert np.all(np.abs(y - dec) == dist)
    mids = (GRID[1:] + GRID[:-1]) / 2
    mc = oracle.e2m1_encode(mids)
    assert np.all((mc & 1) == 0), mc
    assert list(oracle.e2m1_decode(mc)) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert oracle.e2m1_decode(oracle.e2m1_encode([6.0, 6.9, 100.0])).tolist() == [6.0, 6.0, 6.0]
    neg = oracle.e2m1_decode(oracle.e2m1_encode(-y))
    assert np.array_equal(neg, -dec)


def one_column_block(vals):
    w = np.zeros((1, 32, 1), np.float32)
    w[0, :, 0] = vals
    q, e8 = oracle.quantize_rhs_mxfp4(w)
    return q[0, :, 0], int(e8[0, 0, 0])


@pytest.mark.parametrize("amax,code", [
    (6.0, 127), (4.0, 127), (7.99, 127), (3.99, 126), (8.0, 128),
    (0.75, 124), (0.5, 124), (1e-3, 115),          # floor(log2 1e-3) = -10
])
def test_shared_exponent_closed_forms(amax, code):
    v = np.zeros(32, np.float32)
    v[5] = amax
    v[6] = -amax / 3
    _, e = one_column_block(v)
    assert e == code


def test_shared_exponent_property_and_error_bound():
    r = np.random.default_rng(0)
    w = (r.standard_normal((3, 256, 40)) * np.exp(r.uniform(-6, 3, (3, 1, 40)))).astype(np.float32)
    q, e8 = oracle.quantize_rhs_mxfp4(w)
    X = np.ldexp(1.0, e8.astype(np.int64) - 127)                       # [G,K/32,N]
    blocks = np.abs(w.astype(np.float64)).reshape(3, 8, 32, 40).max(axis=2)
    ratio = blocks / X
    assert np.all((ratio >= 4) & (ratio < 8))
    deq = oracle.e2m1_decode(q) * np.repeat(X, 32, axis=1)
    y = np.abs(w / np.repeat(X, 32, axis=1))
    # half the local grid spacing; the clamp region (6, 8) loses up to 2
    bound = np.where(y <= 2, 0.25, np.where(y <= 4, 0.5, np.where(y <= 6, 1.0, 2.0)))
    assert np.all(np.abs(w - deq) <= bound * np.repeat(X, 32, axis=1))


def test_on_grid_blocks_are_exact_and_power_of_two_invariant():
    r = np.random.default_rng(1)
    vals = r.choice(np.concatenate([GRID, -GRID]), size=(2, 64, 8))
    vals[:, 0, :] = 6.0                                  # every block of k 0..31 holds a 6
    vals[:, 32, :] = -4.0                                 # k 32..63: max 4
    w = (vals * 2.0 ** -5).astype(np.float32)
    q, e8 = oracle.quantize_rhs_mxfp4(w)
    X = np.ldexp(1.0, e8.astype(np.int64) - 127)
    assert np.array_equal(oracle.e2m1_decode(q) * np.repeat(X, 32, axis=1), w)
    q2, e82 = oracle.quantize_rhs_mxfp4(w * np.float32(2.0 ** 7))
    assert np.array_equal(q2, q) and np.array_equal(e82.astype(int), e8.astype(int) + 7)


def test_blocks_are_32_along_k_per_column():
    r = np.random.default_rng(2)
    w = (r.standard_normal((2, 128, 16)) * 0.02).astype(np.float32)
    q, e8 = oracle.quantize_rhs_mxfp4(w)
    w2 = w.copy()
    w2[1, 70, 5] = 3.0                                    # block (1, 2, 5) only
    q2, e82 = oracle.quantize_rhs_mxfp4(w2)
    diff_q = np.argwhere(q != q2)
    assert np.all(diff_q[:, 0] == 1) and np.all(diff_q[:, 2] == 5)
    assert np.all((diff_q[:, 1] >= 64) & (diff_q[:, 1] < 96))
    assert [tuple(x) for x in np.argwhere(e8 != e82)] == [(1, 2, 5)]


def test_all_zero_block():
    q, e = one_column_block(np.zeros(32, np.float32))
    assert e == 0 and not q.any()


def fp4_code_of(vals):
    return oracle.e2m1_encode(np.asarray(vals, np.float64))


def test_gmm_unit_scales_equals_fp8_oracle():
    """With every E8M0 scale 1 the MXFP4 product is the FP8 product of the
    same weight values (every E2M1 value is an E4M3 value) with unit 128x128
    scales: the two oracle functions agree bit for bit."""
    r = np.random.default_rng(3)
    M, K, N, gs = 70, 256, 128, np.array([20, 0, 41], np.int32)
    x = r.standard_normal((M, K)).astype(np.float32)
    ql, sl = oracle.quantize_lhs(x)
    vals = r.choice(np.concatenate([GRID, -GRID]), size=(3, K, N))
    q4 = fp4_code_of(vals)
    e8 = np.full((3, K // 32, N), 127, np.uint8)
    q8 = oracle.e4m3_encode(vals.astype(np.float32))
    sr = np.ones((3, K // 128, N // 128), np.float32)
    a = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, gs)
    b = oracle.gmm_fp8(ql, sl, q8, sr, gs)
    assert np.array_equal(a, b)
    assert (a[int(gs.sum()):] == 0).all()


def test_gmm_integer_case_per_32_block_scales():
    """Integer codes, unit LHS scales, one E8M0 per 32-block chosen at random:
    the result is exact, so it must equal sum_b 2^(e_b - 127) * (integer
    matmul of block b) computed with numpy int64 matmuls."""
    r = np.random.default_rng(4)
    M, K, N = 48, 256, 16
    gs = np.array([17, 0, 31], np.int32)
    ints8 = np.arange(-8, 9)
    il = r.choice(ints8, size=(M, K))
    ql = oracle.e4m3_encode(il.astype(np.float32))
    sl = np.ones((M, K // 128), np.float32)
    iw = r.choice(np.array([0, 1, 2, 3, 4, 6, -1, -2, -3, -4, -6]), size=(3, K, N))
    q4 = fp4_code_of(iw)
    e8 = r.integers(124, 131, size=(3, K // 32, N)).astype(np.uint8)
    out = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, gs)
    ref = np.zeros((M, N))
    off = 0
    for g, s in enumerate(gs.tolist()):
        for b in range(K // 32):
            part = il[off:off + s, 32 * b:32 * b + 32].astype(np.int64) @ iw[g, 32 * b:32 * b + 32].astype(np.int64)
            ref[off:off + s] += part * np.ldexp(1.0, e8[g, b].astype(np.int64) - 127)[None, :]
        off += s
    assert np.array_equal(out, ref)


def test_gmm_scale_shift_and_lhs_scale():
    """Raising one column's E8M0 codes by 3 multiplies that column by 8
    exactly; the LHS 1x128 scales multiply each 128-block's contribution."""
    wl = workloads.custom(90, 256, 32, [40, 50], seed=5, w_std=0.05)
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    q4, e8 = oracle.quantize_rhs_mxfp4(workloads.as_f32(wl.w))
    base = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, wl.group_sizes)
    e8b = e8.copy()
    e8b[:, :, 7] += 3
    shifted = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8b, wl.group_sizes)
    assert np.array_equal(shifted[:, 7], base[:, 7] * 8.0)
    others = [c for c in range(32) if c != 7]
    assert np.array_equal(shifted[:, others], base[:, others])
    sl2 = sl.copy()
    sl2[:, 1] = 0.0
    half = oracle.gmm_fp8_mxfp4(ql, sl2, q4, e8, wl.group_sizes)
    ql2 = ql.copy()
    ql2[:, 128:] = 0
    assert np.allclose(half, oracle.gmm_fp8_mxfp4(ql2, sl, q4, e8, wl.group_sizes), rtol=0, atol=0)


def test_gmm_close_to_unquantised_product():
    """Sanity against the fp64 product of the unquantised inputs: the FP8
    LHS and MXFP4 weight errors bound the difference."""
    wl = workloads.custom(200, 512, 64, [80, 0, 120], seed=6, w_std=0.02)
    x, w = workloads.as_f32(wl.x), workloads.as_f32(wl.w)
    ql, sl = oracle.quantize_lhs(x)
    q4, e8 = oracle.quantize_rhs_mxfp4(w)
    out = oracle.gmm_fp8_mxfp4(ql, sl, q4, e8, wl.group_sizes)
    ref = oracle.gmm(x, w, wl.group_sizes)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.2, rel          # E2M1 carries 1 mantissa bit: ~8% relative noise
