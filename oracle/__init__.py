"""CPU oracle for the MoE grouped matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It is a plain, slow fp64 reference of
what the GPU library computes and shares no code with it (the C source in
``gmm_oracle.c`` has its own FP8 codec, quantiser and reference loops).

Functions take numpy arrays (fp32 values; bf16 tensors are passed widened to
fp32, which is exact) and return numpy arrays.  Sources are cited in
``gmm_oracle.c``; all functions are pinned by tests/test_oracle_*.py.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

QBLOCK = 128


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode_array.argtypes = [P, I, P]
    lib.oracle_quantize_lhs.argtypes = [P, I, I, P, P]
    lib.oracle_quantize_rhs.argtypes = [P, I, I, I, P, P]
    lib.oracle_group_offsets.restype = ctypes.c_int
    lib.oracle_group_offsets.argtypes = [P, I, I, P]
    lib.oracle_work_list.restype = ctypes.c_int64
    lib.oracle_work_list.argtypes = [P, I, I, I, P, I]
    lib.oracle_gmm_fp8.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.oracle_gmm_f64.argtypes = [P, P, P, I, I, I, I, P]
    lib.oracle_tgmm_f64.argtypes = [P, P, P, I, I, I, I, P]
    lib.oracle_dx_f64.argtypes = [P, P, P, I, I, I, I, P]
    lib.oracle_swiglu.argtypes = [P, I, I, P]
    lib.oracle_e2m1_decode.restype = ctypes.c_double
    lib.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e2m1_encode.restype = ctypes.c_uint8
    lib.oracle_e2m1_encode.argtypes = [ctypes.c_double]
    lib.oracle_quantize_rhs_mxfp4.argtypes = [P, I, I, I, P, P]
    lib.oracle_gmm_fp8_mxfp4.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.oracle_quant_scales.argtypes = [P, I, P, P]
    lib.oracle_quantize_rhs_int4.argtypes = [P, I, I, I, P, P]
    lib.oracle_gmm_fp8_int4.argtypes = [P, P, P, P, P, I, I, I, I, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().oracle_num_threads()


def e4m3_decode(codes) -> np.ndarray:
    """Values (fp64) of E4M3 codes."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    lut = np.array([lib.oracle_e4m3_decode(c) for c in range(256)])
    return lut[codes]


def e4m3_encode(x) -> np.ndarray:
    """RNE, saturating E4M3 codes of fp32 values."""
    lib = _load()
    x, px = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib.oracle_e4m3_encode_array(px, x.size, out.ctypes.data_as(ctypes.c_void_p))
    return out


def quantize_lhs(x):
    """1x128 quantisation of x [M,K] -> (codes uint8 [M,K], scales f32 [M,K/128])."""
    lib = _load()
    x, px = _c(x, np.float32)
    M, K = x.shape
    assert K % QBLOCK == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // QBLOCK), dtype=np.float32)
    lib.oracle_quantize_lhs(px, M, K, q.ctypes.data_as(ctypes.c_void_p),
                            s.ctypes.data_as(ctypes.c_void_p))
    return q, s


def quantize_rhs(w):
    """128x128 quantisation of w [G,K,N] -> (codes [G,K,N], scales [G,K/128,N/128])."""
    lib = _load()
    w, pw = _c(w, np.float32)
    G, K, N = w.shape
    assert K % QBLOCK == 0 and N % QBLOCK == 0
    q = np.empty((G, K, N), dtype=np.uint8)
    s = np.empty((G, K // QBLOCK, N // QBLOCK), dtype=np.float32)
    lib.oracle_quantize_rhs(pw, G, K, N, q.ctypes.data_as(ctypes.c_void_p),
                            s.ctypes.data_as(ctypes.c_void_p))
    return q, s


def group_offsets(group_sizes, M):
    lib = _load()
    gs, pg = _c(group_sizes, np.int32)
    off = np.empty(gs.size + 1, dtype=np.int64)
    rc = lib.oracle_group_offsets(pg, gs.size, M, off.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("group sizes negative or summing past M")
    return off


def quant_scales(amax):
    """The quantiser's scale pair for block abs-maxima (fp32): (a/448, guarded 1/s)."""
    lib = _load()
    a, pa = _c(amax, np.float32)
    s = np.empty_like(a)
    inv = np.empty_like(a)
    lib.oracle_quant_scales(pa, a.size, s.ctypes.data_as(ctypes.c_void_p),
                            inv.ctypes.data_as(ctypes.c_void_p))
    return s, inv


def work_list(group_sizes, M, tm):
    """(g, tile, row_lo, row_hi) entries of the grouped GEMM, int32 [n,4]."""
    lib = _load()
    gs, pg = _c(group_sizes, np.int32)
    cap = -(-M // tm) + gs.size + 2
    work = np.zeros((cap, 4), dtype=np.int32)
    n = lib.oracle_work_list(pg, gs.size, M, tm, work.ctypes.data_as(ctypes.c_void_p), cap)
    if n < 0:
        raise ValueError("work list overflow")
    return work[:n].copy()


def gmm_fp8(ql, sl, qr, sr, group_sizes):
    """fp64 blockwise-FP8 GMM; ql [M,K], sl [M,K/128], qr [G,K,N] (codes), sr [G,K/128,N/128]."""
    lib = _load()
    ql, pql = _c(ql, np.uint8)
    sl, psl = _c(sl, np.float32)
    qr, pqr = _c(qr, np.uint8)
    sr, psr = _c(sr, np.float32)
    gs, pg = _c(group_sizes, np.int32)
    M, K = ql.shape
    G, K2, N = qr.shape
    assert K == K2 and gs.size == G and int(gs.sum()) <= M
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_gmm_fp8(pql, psl, pqr, psr, pg, M, K, N, G, out.ctypes.data_as(ctypes.c_void_p))
    return out


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 code (low 4 bits) -> fp64 value."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_decode(int(v)) for v in c.ravel()]).reshape(c.shape)


def e2m1_encode(y) -> np.ndarray:
    """fp64 values -> E2M1 codes (nearest, ties to even mantissa, saturating)."""
    lib = _load()
    y = np.asarray(y, dtype=np.float64)
    return np.array([lib.oracle_e2m1_encode(float(v)) for v in y.ravel()],
                    dtype=np.uint8).reshape(y.shape)


def quantize_rhs_mxfp4(w):
    """MXFP4 weights: w [G,K,N] -> (codes [G,K,N] uint8, E8M0 [G,K/32,N] uint8),
    one block of 32 consecutive k per (expert, column)."""
    lib = _load()
    w, pw = _c(w, np.float32)
    G, K, N = w.shape
    assert K % 32 == 0
    q = np.empty((G, K, N), dtype=np.uint8)
    e8 = np.empty((G, K // 32, N), dtype=np.uint8)
    lib.oracle_quantize_rhs_mxfp4(pw, G, K, N, q.ctypes.data_as(ctypes.c_void_p),
                                  e8.ctypes.data_as(ctypes.c_void_p))
    return q, e8


def gmm_fp8_mxfp4(ql, sl, q4, e8, group_sizes):
    """fp64 GMM of FP8 1x128 LHS codes/scales against MXFP4 weights."""
    lib = _load()
    ql, pql = _c(ql, np.uint8)
    sl, psl = _c(sl, np.float32)
    q4, pq4 = _c(q4, np.uint8)
    e8, pe8 = _c(e8, np.uint8)
    gs, pg = _c(group_sizes, np.int32)
    M, K = ql.shape
    G, K2, N = q4.shape
    assert K == K2 and K % QBLOCK == 0 and e8.shape == (G, K // 32, N)
    assert gs.size == G and int(gs.sum()) <= M
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_gmm_fp8_mxfp4(pql, psl, pq4, pe8, pg, M, K, N, G,
                             out.ctypes.data_as(ctypes.c_void_p))
    return out


def quantize_rhs_int4(w):
    """int4 weights: w [G,K,N] -> (codes [G,K,N] int8 in [-8, 7], scales
    [G,K/128,N/128] fp32), one scale per 128x128 block, s = a/7."""
    lib = _load()
    w, pw = _c(w, np.float32)
    G, K, N = w.shape
    assert K % QBLOCK == 0 and N % QBLOCK == 0
    q = np.empty((G, K, N), dtype=np.int8)
    s = np.empty((G, K // QBLOCK, N // QBLOCK), dtype=np.float32)
    lib.oracle_quantize_rhs_int4(pw, G, K, N, q.ctypes.data_as(ctypes.c_void_p),
                                 s.ctypes.data_as(ctypes.c_void_p))
    return q, s


def gmm_fp8_int4(ql, sl, q4, sr, group_sizes):
    """fp64 GMM of FP8 1x128 LHS codes/scales against int4 weights with
    128x128 block scales."""
    lib = _load()
    ql, pql = _c(ql, np.uint8)
    sl, psl = _c(sl, np.float32)
    q4, pq4 = _c(q4, np.int8)
    sr, psr = _c(sr, np.float32)
    gs, pg = _c(group_sizes, np.int32)
    M, K = ql.shape
    G, K2, N = q4.shape
    assert K == K2 and K % QBLOCK == 0 and N % QBLOCK == 0
    assert sr.shape == (G, K // QBLOCK, N // QBLOCK)
    assert gs.size == G and int(gs.sum()) <= M
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_gmm_fp8_int4(pql, psl, pq4, psr, pg, M, K, N, G,
                            out.ctypes.data_as(ctypes.c_void_p))
    return out


def swiglu(gu):
    """fp64 silu(gate) * up of a [M,2N] array whose first N columns are the
    gate projection and the next N the up projection -> [M,N]."""
    lib = _load()
    gu, pg = _c(gu, np.float64)
    M, N2 = gu.shape
    assert N2 % 2 == 0
    out = np.empty((M, N2 // 2), dtype=np.float64)
    lib.oracle_swiglu(pg, M, N2 // 2, out.ctypes.data_as(ctypes.c_void_p))
    return out


def gmm_fp8_swiglu(ql, sl, qr, sr, group_sizes):
    """Fused gate+up FP8 GMM: qr/sr quantise the [G,K,2N] concatenation."""
    return swiglu(gmm_fp8(ql, sl, qr, sr, group_sizes))


def gmm(x, w, group_sizes):
    """fp64 GMM: out[m] = x[m] . w[g(m)]; x [M,K], w [G,K,N]."""
    lib = _load()
    x, px = _c(x, np.float32)
    w, pw = _c(w, np.float32)
    gs, pg = _c(group_sizes, np.int32)
    M, K = x.shape
    G, K2, N = w.shape
    assert K == K2 and gs.size == G and int(gs.sum()) <= M
    out = np.empty((M, N), dtype=np.float64)
    lib.oracle_gmm_f64(px, pw, pg, M, K, N, G, out.ctypes.data_as(ctypes.c_void_p))
    return out


def tgmm(x, dy, group_sizes):
    """fp64 dW[g] = X_g^T dY_g; x [M,K], dy [M,N] -> [G,K,N]."""
    lib = _load()
    x, px = _c(x, np.float32)
    dy, pd = _c(dy, np.float32)
    gs, pg = _c(group_sizes, np.int32)
    M, K = x.shape
    M2, N = dy.shape
    G = gs.size
    assert M == M2 and int(gs.sum()) <= M
    out = np.empty((G, K, N), dtype=np.float64)
    lib.oracle_tgmm_f64(px, pd, pg, M, K, N, G, out.ctypes.data_as(ctypes.c_void_p))
    return out


def gmm_dx(dy, w, group_sizes):
    """fp64 dX[m] = dY[m] . w[g(m)]^T; dy [M,N], w [G,K,N] -> [M,K]."""
    lib = _load()
    dy, pd = _c(dy, np.float32)
    w, pw = _c(w, np.float32)
    gs, pg = _c(group_sizes, np.int32)
    M, N = dy.shape
    G, K, N2 = w.shape
    assert N == N2 and gs.size == G and int(gs.sum()) <= M
    out = np.empty((M, K), dtype=np.float64)
    lib.oracle_dx_f64(pd, pw, pg, M, K, N, G, out.ctypes.data_as(ctypes.c_void_p))
    return out
