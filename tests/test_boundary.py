"""The C ABI on the CPU: the library loads, exports every symbol that
include/gmm.h declares, and rejects bad arguments on the host before any
launch (no call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

import moe_grouped_gemm_gmm_amd as gmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, ALIGN, DTYPE, WORKSPACE = 0, 1, 2, 3, 4, 5
WSB = 256      # the workspace size every grouped call needs today

# fake device addresses: never dereferenced, the checks fail first
A = 0x10000
MIS = 0x10008


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gmm.h")).read()
    text = text.replace("#define GMM_API", "")
    return sorted(set(re.findall(r"GMM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gmm.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) == 23
    assert sorted(names) == sorted(gmm.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.gmm_status_string(0) == b"ok"
    assert lib.gmm_status_string(2) == b"invalid shape"
    assert lib.gmm_status_string(99) == b"unknown status"


def P(x):
    return ctypes.c_void_p(x) if x else None


def fp8(lib, lhs=A, lhs_dt=1, lhs_scale=0, rhs=A, rhs_scale=A, gs=A, M=256, K=256, N=256, G=4,
        out=A, out_dt=1, q=0, s=0, ws=A, wsb=WSB):
    return lib.gmm_fp8_fwd(P(lhs), lhs_dt, P(lhs_scale), P(rhs), P(rhs_scale), P(gs), M, K, N, G,
                           P(out), out_dt, P(q), P(s), P(ws), wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lhs=0), NULL), (dict(rhs=0), NULL), (dict(rhs_scale=0), NULL), (dict(gs=0), NULL),
    (dict(out=0), NULL),
    (dict(lhs=MIS), ALIGN), (dict(out=MIS), ALIGN), (dict(q=MIS, s=A), ALIGN),
    (dict(q=A), NULL),
    (dict(K=200), SHAPE), (dict(N=100), SHAPE), (dict(K=0), SHAPE), (dict(G=0), SHAPE),
    (dict(G=5000), SHAPE), (dict(M=-1), SHAPE),
    (dict(lhs_dt=7), DTYPE), (dict(out_dt=2), DTYPE),
    (dict(lhs_dt=2), NULL),                       # E4M3 lhs needs lhs_scale
    (dict(lhs_dt=2, lhs_scale=A, q=A, s=A), DTYPE),
    (dict(lhs_scale=A), DTYPE),
    (dict(M=0), OK),                              # empty input: nothing to do
    (dict(ws=0), WORKSPACE), (dict(wsb=255), WORKSPACE), (dict(ws=MIS), ALIGN),
    (dict(M=0, ws=0), WORKSPACE),                 # checked before the empty-input return
])
def test_fp8_fwd_rejections(lib, kw, status):
    assert fp8(lib, **kw) == status
    if status:
        assert lib.gmm_last_error()


def fp8_noalloc(lib, lhs=A, lhs_dt=1, lhs_scale=0, rhs=A, rhs_scale=A, gs=A, M=256, K=256, N=256,
                G=4, out=A, out_dt=1, q=0, s=0):
    return lib.gmm_fp8_fwd_noalloc(P(lhs), lhs_dt, P(lhs_scale), P(rhs), P(rhs_scale), P(gs), M, K,
                                   N, G, P(out), out_dt, P(q), P(s), None)


@pytest.mark.parametrize("kw,status", [
    (dict(lhs=0), NULL), (dict(gs=0), NULL), (dict(out=MIS), ALIGN), (dict(q=A), NULL),
    (dict(K=200), SHAPE), (dict(G=0), SHAPE), (dict(M=-1), SHAPE), (dict(lhs_dt=7), DTYPE),
    (dict(lhs_dt=2), NULL), (dict(lhs_scale=A), DTYPE),
    (dict(M=0), OK),                   # nothing to do: returns before touching the device
])
def test_fp8_fwd_noalloc_rejections(lib, kw, status):
    """The no-workspace variant applies gmm_fp8_fwd's checks, before any HIP call."""
    assert fp8_noalloc(lib, **kw) == status


def swiglu(lib, lhs=A, lhs_dt=1, lhs_scale=0, rhs=A, rhs_scale=A, gs=A, M=256, K=256, N=256, G=4,
           out=A, out_dt=1, q=0, s=0, ws=A, wsb=WSB):
    return lib.gmm_fp8_fwd_swiglu(P(lhs), lhs_dt, P(lhs_scale), P(rhs), P(rhs_scale), P(gs), M, K,
                                  N, G, P(out), out_dt, P(q), P(s), P(ws), wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lhs=0), NULL), (dict(rhs=0), NULL), (dict(out=0), NULL),
    (dict(out=MIS), ALIGN), (dict(q=MIS, s=A), ALIGN),
    (dict(q=A), NULL), (dict(s=A), NULL),           # act_q and act_scale together
    (dict(N=128), SHAPE),                           # 256 output columns per tile
    (dict(K=200), SHAPE), (dict(G=0), SHAPE),
    (dict(lhs_dt=2), NULL),                         # E4M3 lhs needs lhs_scale
    (dict(lhs_scale=A), DTYPE), (dict(out_dt=2), DTYPE),
    (dict(M=0), OK), (dict(ws=0), WORKSPACE), (dict(wsb=16), WORKSPACE),
])
def test_fp8_fwd_swiglu_rejections(lib, kw, status):
    assert swiglu(lib, **kw) == status
    if status:
        assert lib.gmm_last_error()


def mx(lib, lhs=A, lhs_dt=1, lhs_scale=0, rhs=A, rhs_scale=A, gs=A, M=256, K=256, N=256, G=4,
       out=A, out_dt=1, ws=A, wsb=WSB):
    return lib.gmm_fp8_mxfp4_fwd(P(lhs), lhs_dt, P(lhs_scale), P(rhs), P(rhs_scale), P(gs), M, K,
                                 N, G, P(out), out_dt, P(ws), wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lhs=0), NULL), (dict(rhs=0), NULL), (dict(rhs_scale=0), NULL), (dict(gs=0), NULL),
    (dict(out=0), NULL), (dict(out=MIS), ALIGN), (dict(rhs_scale=MIS), ALIGN),
    (dict(K=200), SHAPE), (dict(N=100), SHAPE), (dict(G=0), SHAPE), (dict(M=-1), SHAPE),
    (dict(lhs_dt=2), NULL), (dict(lhs_scale=A), DTYPE), (dict(out_dt=2), DTYPE),
    (dict(M=0), OK), (dict(ws=0), WORKSPACE), (dict(ws=MIS), ALIGN),
])
def test_fp8_mxfp4_fwd_rejections(lib, kw, status):
    assert mx(lib, **kw) == status
    if status:
        assert lib.gmm_last_error()


def test_quantize_mxfp4_rejections(lib):
    r = lib.gmm_quantize_rhs_mxfp4
    assert r(P(A), 1, 2, 128, 200, P(A), P(A), None) == SHAPE
    assert r(P(A), 1, 2, 100, 128, P(A), P(A), None) == SHAPE
    assert r(P(A), 1, 0, 128, 128, P(A), P(A), None) == SHAPE
    assert r(P(A), 2, 2, 128, 128, P(A), P(A), None) == DTYPE
    assert r(P(A), 0, 2, 128, 128, None, P(A), None) == NULL
    assert r(P(A), 0, 2, 128, 128, P(A), P(MIS), None) == ALIGN


def i4(lib, lhs=A, lhs_dt=1, lhs_scale=0, rhs=A, rhs_scale=A, gs=A, M=256, K=256, N=256, G=4,
       out=A, out_dt=1, ws=A, wsb=WSB):
    return lib.gmm_fp8_int4_fwd(P(lhs), lhs_dt, P(lhs_scale), P(rhs), P(rhs_scale), P(gs), M, K,
                                N, G, P(out), out_dt, P(ws), wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lhs=0), NULL), (dict(rhs=0), NULL), (dict(rhs_scale=0), NULL), (dict(gs=0), NULL),
    (dict(out=0), NULL), (dict(out=MIS), ALIGN), (dict(rhs_scale=MIS), ALIGN),
    (dict(K=200), SHAPE), (dict(N=100), SHAPE), (dict(G=0), SHAPE), (dict(M=-1), SHAPE),
    (dict(lhs_dt=2), NULL), (dict(lhs_scale=A), DTYPE), (dict(out_dt=2), DTYPE), (dict(lhs_dt=5), DTYPE),
    (dict(M=0), OK), (dict(ws=0), WORKSPACE), (dict(ws=MIS), ALIGN), (dict(wsb=8), WORKSPACE),
])
def test_fp8_int4_fwd_rejections(lib, kw, status):
    assert i4(lib, **kw) == status
    if status:
        assert lib.gmm_last_error()


def test_int4_quantize_and_pack_rejections(lib):
    r = lib.gmm_quantize_rhs_int4
    assert r(P(A), 1, 2, 128, 200, P(A), P(A), None) == SHAPE
    assert r(P(A), 1, 2, 100, 128, P(A), P(A), None) == SHAPE
    assert r(P(A), 1, 0, 128, 128, P(A), P(A), None) == SHAPE
    assert r(P(A), 2, 2, 128, 128, P(A), P(A), None) == DTYPE
    assert r(P(A), 0, 2, 128, 128, None, P(A), None) == NULL
    assert r(P(A), 0, 2, 128, 128, P(A), P(MIS), None) == ALIGN
    p = lib.gmm_pack_rhs_int4
    B = A + 0x100000
    assert p(P(A), 2, 128, 200, P(B), None) == SHAPE
    assert p(P(A), 2, 100, 128, P(B), None) == SHAPE
    assert p(P(A), 0, 128, 128, P(B), None) == SHAPE
    assert p(None, 2, 128, 128, P(B), None) == NULL
    assert p(P(A), 2, 128, 128, P(MIS), None) == ALIGN
    assert p(P(A), 2, 128, 128, P(A + 4096), None) == SHAPE       # packed overlaps q
    assert b"overlaps" in lib.gmm_last_error()


def test_quantize_rejections(lib):
    q = lib.gmm_quantize_lhs
    assert q(P(A), 1, 16, 100, P(A), P(A), None) == SHAPE
    assert q(P(A), 2, 16, 128, P(A), P(A), None) == DTYPE
    assert q(None, 1, 16, 128, P(A), P(A), None) == NULL
    assert q(P(A), 1, 16, 128, P(MIS), P(A), None) == ALIGN
    assert q(P(A), 1, 0, 128, P(A), P(A), None) == OK
    r = lib.gmm_quantize_rhs
    assert r(P(A), 1, 2, 128, 200, P(A), P(A), None) == SHAPE
    assert r(P(A), 1, 0, 128, 128, P(A), P(A), None) == SHAPE
    assert r(P(A), 0, 2, 128, 128, None, P(A), None) == NULL


def test_bf16_rejections(lib):
    f, t, d = lib.gmm_bf16_fwd, lib.tgmm_bf16, lib.gmm_bf16_dx
    W = (P(A), WSB, None)
    assert f(P(A), P(A), P(A), 64, 100, 128, 2, P(A), 1, *W) == SHAPE
    assert f(P(A), P(A), P(A), 64, 128, 64, 2, P(A), 1, *W) == SHAPE
    assert f(P(A), P(A), P(A), 64, 128, 128, 2, P(A), 3, *W) == DTYPE
    assert f(P(A), None, P(A), 64, 128, 128, 2, P(A), 1, *W) == NULL
    assert f(P(A), P(A), P(A), 0, 128, 128, 2, P(A), 1, *W) == OK
    assert f(P(A), P(A), P(A), 64, 128, 128, 2, P(A), 1, None, WSB, None) == WORKSPACE
    assert t(P(A), P(A), P(A), 64, 64, 128, 2, P(A), 1, *W) == SHAPE
    assert t(P(A), P(MIS), P(A), 64, 128, 128, 2, P(A), 1, *W) == ALIGN
    assert t(P(A), P(A), P(A), 64, 128, 128, 2, P(A), 1, P(A), 8, None) == WORKSPACE
    assert d(P(A), P(A), P(A), 64, 128, 96, 2, P(A), 1, *W) == SHAPE
    assert d(P(A), P(A), P(A), 64, 128, 128, 0, P(A), 1, *W) == SHAPE
    assert d(P(A), P(A), P(A), 64, 128, 128, 2, P(A), 1, P(MIS), WSB, None) == ALIGN


def test_metadata_rejections(lib):
    m = lib.gmm_group_metadata
    W = (P(A), WSB, None)
    assert m(P(A), 4, 100, 100, P(A), P(A), 100, P(A), *W) == SHAPE   # tile not a multiple of 16
    assert m(P(A), 4, 100, 2048, P(A), P(A), 100, P(A), *W) == SHAPE  # tile above 1024
    assert m(P(A), 4, 1000, 128, P(A), P(A), 5, P(A), *W) == SHAPE    # capacity too small
    assert m(P(A), 4, 1000, 128, P(A), None, 20, P(A), *W) == NULL
    assert m(P(A), 4, 1000, 128, P(A), P(A), 20, P(A), None, 0, None) == WORKSPACE


def test_workspace_bytes(lib):
    for op in range(8):
        assert lib.gmm_workspace_bytes(op, 65536, 2048, 512, 256) == WSB
    assert lib.gmm_workspace_bytes(8, 1, 128, 128, 1) == 0
    assert lib.gmm_workspace_bytes(-1, 1, 128, 128, 1) == 0
    assert lib.gmm_status_string(WORKSPACE) == b"workspace missing or too small"


def test_device_status_rejections(lib):
    st = ctypes.c_int32(0)
    assert lib.gmm_device_status(None, ctypes.byref(st), None) == NULL
    assert lib.gmm_device_status(P(MIS), ctypes.byref(st), None) == ALIGN
    assert lib.gmm_device_status(P(A), None, None) == NULL


def test_pack_rhs_rejections(lib):
    p = lib.gmm_pack_rhs
    assert p(P(A), 2, 128, 200, P(A), None) == SHAPE
    assert p(P(A), 2, 100, 128, P(A), None) == SHAPE
    assert p(P(A), 0, 128, 128, P(A), None) == SHAPE
    assert p(P(A), 5000, 128, 128, P(A), None) == SHAPE
    assert p(None, 2, 128, 128, P(A), None) == NULL
    assert p(P(A), 2, 128, 128, P(MIS), None) == ALIGN


def test_quant_scales_rejections(lib):
    q = lib.gmm_quant_scales
    assert q(P(A), -1, P(A), P(A), None) == SHAPE
    assert q(None, 4, P(A), P(A), None) == NULL
    assert q(P(A), 4, P(A), P(MIS), None) == ALIGN
    assert q(P(A), 0, P(A), P(A), None) == OK


def test_binding_raises_on_error(lib):
    with pytest.raises(gmm.GmmError) as e:
        gmm._check(SHAPE)
    assert e.value.status == SHAPE


def test_tile_config_rejections(lib):
    c = gmm.TileConfig(kernel=1, waves=16)
    assert lib.gmm_set_tile_config(0, ctypes.byref(c)) == SHAPE      # metadata has no tiles
    assert lib.gmm_set_tile_config(8, ctypes.byref(c)) == SHAPE
    bad = gmm.TileConfig(kernel=4)
    assert lib.gmm_set_tile_config(1, ctypes.byref(bad)) == SHAPE
    assert lib.gmm_get_tile_config(1, 256, 256, 256, 4, 1, 1, None) == NULL
    out = gmm.TileConfig()
    assert lib.gmm_get_tile_config(1, 256, 256, 256, 4, 1, 2, ctypes.byref(out)) == DTYPE
    # a configuration that does not fit a call's shape makes that call fail before launching
    assert lib.gmm_set_tile_config(1, ctypes.byref(gmm.TileConfig(kernel=1))) == OK
    try:
        assert fp8(lib, N=256) == SHAPE                   # 48 x 512 tiles need N % 512 == 0
        assert b"does not fit" in lib.gmm_last_error()
    finally:
        assert lib.gmm_set_tile_config(1, None) == OK
    assert fp8(lib, N=256, M=0) == OK


def test_probe_rejections(lib):
    p = lib.gmm_probe_stream_read
    assert p(P(A), 1000, P(A), None) == SHAPE
    assert p(P(A), 0, P(A), None) == SHAPE
    assert p(None, 65536, P(A), None) == NULL
    assert p(P(A), 65536, P(MIS), None) == ALIGN
