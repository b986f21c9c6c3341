"""Pins of the oracle's grouped matmuls (FP8 forward, bf16 forward, tgmm, dX)
and of its work list, against exact rational arithmetic, numpy fp64 dense
products, closed forms and invariants.

Definitions: "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4",
section 3.7.2 (one GEMM per expert over its rows); "GEMM Kernel 性能优化十问",
Q3 (per-subchannel scale and accumulate), Q4 (tgmm reduces over M), Q5
(bf16 backward); "实现差距：GMM Kernel（V1 vs V2）", sections 2.1 and 3.3
(per-block dot, rescale by LHS and RHS scales, accumulate) and 3.6 (rows
past the last group are zero).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def rand_codes(r, shape):
    """Random finite E4M3 codes (no NaN)."""
    c = r.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def dense_fp8_per_group(ql, sl, qr, sr, gs):
    """numpy fp64: per group, per 128-block dense products of decoded codes."""
    M, K = ql.shape
    G, _, N = qr.shape
    dl = oracle.e4m3_decode(ql)
    dr = oracle.e4m3_decode(qr)
    out = np.zeros((M, N))
    o = 0
    for g in range(G):
        rows = slice(o, o + gs[g])
        for b in range(K // 128):
            ks = slice(128 * b, 128 * b + 128)
            part = dl[rows, ks] @ dr[g, ks, :]
            col_scale = np.repeat(sr[g, b, :].astype(np.float64), 128)
            out[rows] += part * sl[rows, b:b + 1].astype(np.float64) * col_scale[None, :]
        o += gs[g]
    return out


# ------------------------------------------------------------- FP8 ----------

@pytest.mark.parametrize("M,K,N,gs", [
    (1, 128, 128, [1]),
    (7, 256, 128, [3, 0, 4]),
    (9, 128, 256, [0, 5, 2]),   # two empty-ish groups, tail of 2 rows
])
def test_fp8_bruteforce_rational(M, K, N, gs):
    r = np.random.default_rng(M * 131 + K)
    G = len(gs)
    ql, qr = rand_codes(r, (M, K)), rand_codes(r, (G, K, N))
    sl = r.uniform(0.01, 2.0, size=(M, K // 128)).astype(np.float32)
    sr = r.uniform(0.01, 2.0, size=(G, K // 128, N // 128)).astype(np.float32)
    out = oracle.gmm_fp8(ql, sl, qr, sr, np.array(gs, np.int32))
    val = {c: Fraction(float(oracle.e4m3_decode(np.array([c], np.uint8))[0])) for c in range(256)
           if (c & 0x7F) != 0x7F}
    cols = list(range(0, N, 37)) + [N - 1]
    m = 0
    for g in range(G):
        for _ in range(gs[g]):
            for n in cols:
                ref = Fraction(0)
                for b in range(K // 128):
                    part = sum(val[int(ql[m, k])] * val[int(qr[g, k, n])] for k in range(128 * b, 128 * b + 128))
                    ref += part * Fraction(float(sl[m, b])) * Fraction(float(sr[g, b, n // 128]))
                assert abs(Fraction(out[m, n]) - ref) <= abs(ref) * Fraction(1, 2 ** 50)
            m += 1
    assert (out[m:] == 0).all()


def test_fp8_single_group_matches_numpy_dense():
    r = np.random.default_rng(3)
    M, K, N = 70, 384, 256
    ql, qr = rand_codes(r, (M, K)), rand_codes(r, (1, K, N))
    sl = r.uniform(0.001, 1.0, size=(M, K // 128)).astype(np.float32)
    sr = r.uniform(0.001, 1.0, size=(1, K // 128, N // 128)).astype(np.float32)
    gs = np.array([M], np.int32)
    out = oracle.gmm_fp8(ql, sl, qr, sr, gs)
    ref = dense_fp8_per_group(ql, sl, qr, sr, gs)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-300)


def test_fp8_grouped_matches_numpy_per_group():
    r = np.random.default_rng(4)
    gs = np.array([5, 0, 17, 1, 0, 9], np.int32)
    M, K, N = 40, 256, 256
    G = gs.size
    ql, qr = rand_codes(r, (M, K)), rand_codes(r, (G, K, N))
    sl = r.uniform(0.001, 1.0, size=(M, K // 128)).astype(np.float32)
    sr = r.uniform(0.001, 1.0, size=(G, K // 128, N // 128)).astype(np.float32)
    out = oracle.gmm_fp8(ql, sl, qr, sr, gs)
    ref = dense_fp8_per_group(ql, sl, qr, sr, gs)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-300)
    assert (out[gs.sum():] == 0).all()


def test_fp8_exact_integer_case():
    """Unit scales and small-integer codes: every sum is an exact integer."""
    r = np.random.default_rng(5)
    ints = np.array([-8, -7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7, 8], np.float32)
    code_of = {int(v): int(c) for v, c in zip(ints, oracle.e4m3_encode(ints))}
    M, K, N, gs = 33, 256, 128, np.array([10, 0, 23], np.int32)
    il = r.integers(-8, 9, size=(M, K))
    ir = r.integers(-8, 9, size=(3, K, N))
    ql = np.vectorize(code_of.get)(il).astype(np.uint8)
    qr = np.vectorize(code_of.get)(ir).astype(np.uint8)
    out = oracle.gmm_fp8(ql, np.ones((M, 2), np.float32), qr, np.ones((3, 2, 1), np.float32), gs)
    ref = np.zeros((M, N), np.int64)
    ref[:10] = il[:10] @ ir[0]
    ref[10:] = il[10:] @ ir[2]
    assert np.array_equal(out, ref.astype(np.float64))


def test_fp8_concatenation_of_groups():
    r = np.random.default_rng(6)
    gs = np.array([12, 7, 0, 21], np.int32)
    M, K, N = 45, 256, 128
    G = gs.size
    ql, qr = rand_codes(r, (M, K)), rand_codes(r, (G, K, N))
    sl = r.uniform(0.01, 1.0, size=(M, 2)).astype(np.float32)
    sr = r.uniform(0.01, 1.0, size=(G, 2, 1)).astype(np.float32)
    out = oracle.gmm_fp8(ql, sl, qr, sr, gs)
    o = 0
    for g in range(G):
        rows = slice(o, o + gs[g])
        single = oracle.gmm_fp8(ql[rows], sl[rows], qr[g:g + 1], sr[g:g + 1], gs[g:g + 1])
        assert np.array_equal(out[rows], single)
        o += gs[g]


def test_fp8_empty_group_never_read_and_tail_zero():
    r = np.random.default_rng(7)
    gs = np.array([6, 9], np.int32)
    M, K, N = 20, 128, 128
    ql, qr = rand_codes(r, (M, K)), rand_codes(r, (2, K, N))
    sl = r.uniform(0.01, 1.0, size=(M, 1)).astype(np.float32)
    sr = r.uniform(0.01, 1.0, size=(2, 1, 1)).astype(np.float32)
    base = oracle.gmm_fp8(ql, sl, qr, sr, gs)
    # insert an empty expert whose weights are NaN codes and NaN scales
    qr3 = np.concatenate([qr[:1], np.full((1, K, N), 0x7F, np.uint8), qr[1:]])
    sr3 = np.concatenate([sr[:1], np.full((1, 1, 1), np.nan, np.float32), sr[1:]])
    out = oracle.gmm_fp8(ql, sl, qr3, sr3, np.array([6, 0, 9], np.int32))
    assert np.array_equal(out, base)
    assert (out[15:] == 0).all() and np.isfinite(out).all()


def test_fp8_end_to_end_quantised_close_to_unquantised():
    """Quantisation noise only: SQNR against the unquantised fp64 product is
    in the pages' 'good' band (> 20 dB; typically ~28-30 dB for N(0,1))."""
    r = np.random.default_rng(8)
    M, K, N = 64, 512, 256
    gs = np.array([30, 34], np.int32)
    x = r.standard_normal((M, K), dtype=np.float32)
    w = r.standard_normal((2, K, N), dtype=np.float32) * np.float32(0.02)
    ql, sl = oracle.quantize_lhs(x)
    qr, sr = oracle.quantize_rhs(w)
    out = oracle.gmm_fp8(ql, sl, qr, sr, gs)
    ref = oracle.gmm(x, w, gs)
    sqnr = 10 * np.log10(np.sum(ref ** 2) / np.sum((ref - out) ** 2))
    assert sqnr > 20.0


# ---------------------------------------------------- bf16 fwd / tgmm / dX --

def _groups(r, M, G, tail=0):
    cuts = np.sort(r.integers(0, M - tail + 1, size=G - 1))
    gs = np.diff(np.concatenate([[0], cuts, [M - tail]])).astype(np.int32)
    return gs


def _ints(r, shape, lim=8):
    return r.integers(-lim, lim + 1, size=shape).astype(np.float32)


def test_gmm_f64_matches_numpy_and_bruteforce():
    r = np.random.default_rng(11)
    M, K, N, G = 37, 96, 40, 4
    gs = np.array([10, 0, 20, 3], np.int32)
    x = r.standard_normal((M, K), dtype=np.float32)
    w = r.standard_normal((G, K, N), dtype=np.float32)
    out = oracle.gmm(x, w, gs)
    o = 0
    for g in range(G):
        rows = slice(o, o + gs[g])
        assert np.allclose(out[rows], x[rows].astype(np.float64) @ w[g].astype(np.float64), rtol=1e-12, atol=1e-12)
        o += gs[g]
    assert (out[o:] == 0).all()
    m, n = 12, 7                                      # brute force one element, exact
    ref = sum(Fraction(float(x[m, k])) * Fraction(float(w[2, k, n])) for k in range(K))
    assert abs(Fraction(out[m, n]) - ref) <= abs(ref) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


def test_tgmm_sum_equals_dense_and_empty_zero():
    r = np.random.default_rng(12)
    M, K, N = 50, 64, 48
    gs = np.array([0, 20, 0, 25, 5, 0], np.int32)
    x = r.standard_normal((M, K), dtype=np.float32)
    dy = r.standard_normal((M, N), dtype=np.float32)
    dw = oracle.tgmm(x, dy, gs)
    assert np.allclose(dw.sum(0), x.astype(np.float64).T @ dy.astype(np.float64), rtol=1e-12, atol=1e-10)
    for g in np.nonzero(gs == 0)[0]:
        assert (dw[g] == 0).all()
    o = 0
    for g in range(gs.size):
        rows = slice(o, o + gs[g])
        assert np.allclose(dw[g], x[rows].astype(np.float64).T @ dy[rows].astype(np.float64), rtol=1e-12, atol=1e-10)
        o += gs[g]


def test_tgmm_tail_rows_ignored():
    r = np.random.default_rng(13)
    M, K, N = 30, 16, 16
    gs = np.array([10, 12], np.int32)
    x = r.standard_normal((M, K), dtype=np.float32)
    dy = r.standard_normal((M, N), dtype=np.float32)
    a = oracle.tgmm(x, dy, gs)
    x2 = x.copy()
    x2[22:] = 1e30
    assert np.array_equal(oracle.tgmm(x2, dy, gs), a)


def test_dx_matches_numpy_and_tail_zero():
    r = np.random.default_rng(14)
    M, K, N = 41, 64, 80
    gs = np.array([7, 0, 30], np.int32)
    dy = r.standard_normal((M, N), dtype=np.float32)
    w = r.standard_normal((3, K, N), dtype=np.float32)
    dx = oracle.gmm_dx(dy, w, gs)
    o = 0
    for g in range(3):
        rows = slice(o, o + gs[g])
        assert np.allclose(dx[rows], dy[rows].astype(np.float64) @ w[g].astype(np.float64).T, rtol=1e-12, atol=1e-10)
        o += gs[g]
    assert (dx[o:] == 0).all()


def test_exact_small_integers_fwd_tgmm_dx():
    r = np.random.default_rng(15)
    M, K, N = 40, 64, 32
    gs = np.array([15, 0, 25], np.int32)
    x, dy = _ints(r, (M, K)), _ints(r, (M, N))
    w = _ints(r, (3, K, N))
    xi, dyi, wi = x.astype(np.int64), dy.astype(np.int64), w.astype(np.int64)
    fwd = np.zeros((M, N), np.int64)
    fwd[:15] = xi[:15] @ wi[0]
    fwd[15:] = xi[15:] @ wi[2]
    assert np.array_equal(oracle.gmm(x, w, gs), fwd.astype(np.float64))
    dw = np.zeros((3, K, N), np.int64)
    dw[0] = xi[:15].T @ dyi[:15]
    dw[2] = xi[15:].T @ dyi[15:]
    assert np.array_equal(oracle.tgmm(x, dy, gs), dw.astype(np.float64))
    dx = np.zeros((M, K), np.int64)
    dx[:15] = dyi[:15] @ wi[0].T
    dx[15:] = dyi[15:] @ wi[2].T
    assert np.array_equal(oracle.gmm_dx(dy, w, gs), dx.astype(np.float64))


def test_adjoint_identity_ties_fwd_dx_tgmm():
    """<GMM(X,W), dY> = <X, dX> = sum_g <W_g, dW_g> for the same groups."""
    r = np.random.default_rng(16)
    M, K, N = 64, 48, 40
    gs = np.array([20, 0, 30, 4], np.int32)   # 10 tail rows
    x = r.standard_normal((M, K), dtype=np.float32)
    w = r.standard_normal((4, K, N), dtype=np.float32)
    dy = r.standard_normal((M, N), dtype=np.float32)
    y = oracle.gmm(x, w, gs)
    dx = oracle.gmm_dx(dy, w, gs)
    dw = oracle.tgmm(x, dy, gs)
    a = np.sum(y * dy.astype(np.float64))
    b = np.sum(x.astype(np.float64) * dx)
    c = np.sum(w.astype(np.float64) * dw)
    scale = np.sqrt(np.sum(y ** 2) * np.sum(dy.astype(np.float64) ** 2))
    assert abs(a - b) <= 1e-10 * scale and abs(a - c) <= 1e-10 * scale


# ------------------------------------------------------------ work list -----

def bruteforce_work(gs, M, tm):
    """Scan every row; collect (g, t) -> [min row, max row + 1].  Rows are dealt
    to groups in order, a negative size dealing none; the rows left below M
    belong to no group (g = G); rows dealt past M do not exist."""
    dealt = [np.full(max(s, 0), g) for g, s in enumerate(gs)]
    gid = np.concatenate(dealt + [np.full(M, len(gs))]).astype(int)[:M]
    seen = {}
    for row in range(M):
        key = (int(gid[row]), row // tm)
        lo, hi = seen.get(key, (row, row + 1))
        seen[key] = (min(lo, row), max(hi, row + 1))
    return sorted([(g, t, lo, hi) for (g, t), (lo, hi) in seen.items()])


@pytest.mark.parametrize("gs,M,tm", [
    ([512], 512, 128),
    ([0, 0, 300, 0], 300, 128),
    ([1, 1, 1, 1], 10, 4),
    ([127, 1, 128, 0, 129], 400, 128),
    ([0, 0, 0], 5, 2),
    ([3, 5, 0, 7], 15, 16),
])
def test_work_list_bruteforce(gs, M, tm):
    gs = np.array(gs, np.int32)
    wl = oracle.work_list(gs, M, tm)
    assert sorted(map(tuple, wl.tolist())) == bruteforce_work(gs.tolist(), M, tm)
    # group-major order, tail (g == G) last
    assert wl[:, 0].tolist() == sorted(wl[:, 0].tolist())


@pytest.mark.parametrize("gs,M,tm", [
    ([128, 128], 128, 128),          # sizes sum past M: group 1 has no rows left
    ([100, 100, 100], 250, 64),      # group 2 is cut at M
    ([5, -3, 7], 20, 16),            # a negative size deals no rows
    ([-5, 0, 30], 16, 16),           # negative first, then past M
    ([0, 2**31 - 1, 9], 64, 16),     # a size far beyond M
])
def test_work_list_outside_contract(gs, M, tm):
    """Out-of-contract group sizes: rows stay inside [0, M) (the boundary's
    reading, gmm.h), checked against the row scan above."""
    gs = np.array(gs, np.int32)
    wl = oracle.work_list(gs, M, tm)
    assert sorted(map(tuple, wl.tolist())) == bruteforce_work(gs.tolist(), M, tm)
    assert (wl[:, 2] >= 0).all() and (wl[:, 3] <= M).all() and (wl[:, 2] < wl[:, 3]).all()
    assert len(wl) <= -(-M // tm) + gs.size + 1


def test_work_list_random_and_bound():
    r = np.random.default_rng(17)
    for trial in range(30):
        G = int(r.integers(1, 40))
        M = int(r.integers(1, 3000))
        tm = int(r.choice([16, 32, 64, 128, 256]))
        gs = _groups(r, M, G, tail=int(r.integers(0, min(M, 50))))
        wl = oracle.work_list(gs, M, tm)
        assert sorted(map(tuple, wl.tolist())) == bruteforce_work(gs.tolist(), M, tm)
        assert len(wl) <= -(-M // tm) + G + 1
