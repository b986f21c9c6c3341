"""Python binding of the gfx950 grouped-matmul library (libgmm.so, include/gmm.h).

Argument marshalling only: every function checks nothing that the C ABI does
not already check, allocates outputs with torch (device memory), and calls
the library on torch's current stream.  All compute runs in the HIP kernels;
there is no CPU or eager-PyTorch fallback.  If libgmm.so is missing or cannot
be loaded, every call raises.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgmm.so")

GMM_F32, GMM_BF16, GMM_E4M3 = 0, 1, 2
GMM_MAX_GROUPS = 4096
# operations (gmm_workspace_bytes) and device status bits (gmm_device_status)
(OP_METADATA, OP_FP8_FWD, OP_FP8_FWD_SWIGLU, OP_FP8_MXFP4_FWD, OP_BF16_FWD, OP_TGMM,
 OP_DX, OP_FP8_INT4_FWD) = range(8)
DEV_SUM_GT_M, DEV_NEGATIVE_SIZE = 1, 2
EXPORTS = ("gmm_status_string", "gmm_last_error", "gmm_workspace_bytes", "gmm_device_status",
           "gmm_set_tile_config", "gmm_get_tile_config", "gmm_probe_stream_read",
           "gmm_group_metadata", "gmm_quantize_lhs", "gmm_quantize_rhs", "gmm_pack_rhs",
           "gmm_quant_scales", "gmm_fp8_fwd", "gmm_fp8_fwd_swiglu", "gmm_bf16_fwd", "tgmm_bf16",
           "gmm_bf16_dx", "gmm_quantize_rhs_mxfp4", "gmm_fp8_mxfp4_fwd", "gmm_fp8_fwd_noalloc",
           "gmm_quantize_rhs_int4", "gmm_pack_rhs_int4", "gmm_fp8_int4_fwd")

_lib = None

TILE_FIELDS = ("kernel", "waves", "tile_m", "tile_n", "depth", "residency", "placement")


class TileConfig(ctypes.Structure):
    """gmm_tile_config (include/gmm.h); 0 in an override means the library's choice."""
    _fields_ = [(f, ctypes.c_int32) for f in TILE_FIELDS]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f in TILE_FIELDS}


class GmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("gmm status %d: %s" % (status, message))
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgmm.so (raises if it is absent: build it with build.py first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libgmm.so not found at %s; run moe_grouped_gemm_gmm_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.gmm_status_string.restype = ctypes.c_char_p
    lib.gmm_status_string.argtypes = [I]
    lib.gmm_last_error.restype = ctypes.c_char_p
    lib.gmm_last_error.argtypes = []
    lib.gmm_workspace_bytes.restype = SZ
    lib.gmm_workspace_bytes.argtypes = [I, I64, I64, I64, I64]
    lib.gmm_device_status.argtypes = [P, P, P]
    lib.gmm_set_tile_config.argtypes = [I, P]
    lib.gmm_probe_stream_read.argtypes = [P, I64, P, P]
    lib.gmm_get_tile_config.argtypes = [I, I64, I64, I64, I64, I, I, P]
    lib.gmm_group_metadata.argtypes = [P, I64, I64, I64, P, P, I64, P, P, SZ, P]
    lib.gmm_quantize_lhs.argtypes = [P, I, I64, I64, P, P, P]
    lib.gmm_quantize_rhs.argtypes = [P, I, I64, I64, I64, P, P, P]
    lib.gmm_pack_rhs.argtypes = [P, I64, I64, I64, P, P]
    lib.gmm_quant_scales.argtypes = [P, I64, P, P, P]
    lib.gmm_fp8_fwd.argtypes = [P, I, P, P, P, P, I64, I64, I64, I64, P, I, P, P, P, SZ, P]
    lib.gmm_fp8_fwd_noalloc.argtypes = [P, I, P, P, P, P, I64, I64, I64, I64, P, I, P, P, P]
    lib.gmm_fp8_fwd_swiglu.argtypes = [P, I, P, P, P, P, I64, I64, I64, I64, P, I, P, P, P, SZ, P]
    lib.gmm_bf16_fwd.argtypes = [P, P, P, I64, I64, I64, I64, P, I, P, SZ, P]
    lib.tgmm_bf16.argtypes = [P, P, P, I64, I64, I64, I64, P, I, P, SZ, P]
    lib.gmm_bf16_dx.argtypes = [P, P, P, I64, I64, I64, I64, P, I, P, SZ, P]
    lib.gmm_quantize_rhs_mxfp4.argtypes = [P, I, I64, I64, I64, P, P, P]
    lib.gmm_fp8_mxfp4_fwd.argtypes = [P, I, P, P, P, P, I64, I64, I64, I64, P, I, P, SZ, P]
    lib.gmm_quantize_rhs_int4.argtypes = [P, I, I64, I64, I64, P, P, P]
    lib.gmm_pack_rhs_int4.argtypes = [P, I64, I64, I64, P, P]
    lib.gmm_fp8_int4_fwd.argtypes = [P, I, P, P, P, P, I64, I64, I64, I64, P, I, P, SZ, P]
    for name in EXPORTS[3:]:
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        lib = load_library()
        raise GmmError(rc, lib.gmm_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


_DT = {torch.float32: GMM_F32, torch.bfloat16: GMM_BF16, torch.uint8: GMM_E4M3,
       torch.float8_e4m3fn: GMM_E4M3}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return _DT[t.dtype]


def workspace_bytes(op: int, M: int, K: int, N: int, G: int) -> int:
    """Bytes of workspace the grouped call `op` (OP_*) needs for this shape."""
    return int(load_library().gmm_workspace_bytes(op, M, K, N, G))


def workspace(op: int, M: int, K: int, N: int, G: int, device) -> torch.Tensor:
    """A workspace tensor (uint8, device memory) for the grouped call `op`."""
    return torch.empty(max(workspace_bytes(op, M, K, N, G), 16), dtype=torch.uint8, device=device)


def device_status(ws: torch.Tensor) -> int:
    """The device status word the last grouped call wrote into ws (0, or an OR
    of DEV_SUM_GT_M and DEV_NEGATIVE_SIZE); synchronises with the current stream."""
    lib = load_library()
    out = ctypes.c_int32(-1)
    _check(lib.gmm_device_status(_ptr(ws), ctypes.byref(out), _stream(ws)))
    return int(out.value)


def probe_stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Platform probe: stream-read all of buf (a multiple of 64 KB) on the
    current stream; sink holds buf.nbytes / 65536 uint32 words."""
    lib = load_library()
    _check(lib.gmm_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                     _stream(buf)))


def set_tile_config(op: int, cfg: Optional[dict]) -> None:
    """Force a tile configuration for op (OP_*), process-wide; None restores the
    library's choice.  Keys: TILE_FIELDS (missing keys = the library's choice)."""
    lib = load_library()
    if cfg is None:
        _check(lib.gmm_set_tile_config(op, None))
        return
    unknown = set(cfg) - set(TILE_FIELDS)
    if unknown:
        raise ValueError("unknown tile fields %s" % sorted(unknown))
    c = TileConfig(**{f: int(cfg.get(f, 0)) for f in TILE_FIELDS})
    _check(lib.gmm_set_tile_config(op, ctypes.byref(c)))


def get_tile_config(op: int, M: int, K: int, N: int, G: int, lhs_dtype: int = GMM_BF16,
                    out_dtype: int = GMM_BF16) -> dict:
    """The configuration a call of op on this shape would run."""
    lib = load_library()
    c = TileConfig()
    _check(lib.gmm_get_tile_config(op, M, K, N, G, lhs_dtype, out_dtype, ctypes.byref(c)))
    return c.as_dict()


def _ws(ws: Optional[torch.Tensor], op: int, M: int, K: int, N: int, G: int, device):
    if ws is None:
        ws = workspace(op, M, K, N, G, device)
    return ws, _ptr(ws), ws.numel() * ws.element_size()


def gmm_group_metadata(group_sizes: torch.Tensor, M: int, tile_m: int = 128,
                       ws: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Device work list of the grouped kernels: (offsets [G+1], work [cap,4], num_work [1])."""
    lib = load_library()
    G = group_sizes.numel()
    cap = -(-M // tile_m) + G + 1
    dev = group_sizes.device
    offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    work = torch.empty((cap, 4), dtype=torch.int32, device=dev)
    num = torch.empty(1, dtype=torch.int32, device=dev)
    ws, wsp, wsb = _ws(ws, OP_METADATA, M, 0, 0, G, dev)
    _check(lib.gmm_group_metadata(_ptr(group_sizes), G, M, tile_m, _ptr(offsets), _ptr(work),
                                  cap, _ptr(num), wsp, wsb, _stream(group_sizes)))
    return offsets, work, num


def gmm_quantize_lhs(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """1x128 quantisation of x [M,K] (bf16/fp32) -> (codes uint8 [M,K], scales f32 [M,K/128])."""
    lib = load_library()
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, max(K // 128, 0)), dtype=torch.float32, device=x.device)
    _check(lib.gmm_quantize_lhs(_ptr(x), _dt(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def gmm_quantize_rhs(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """128x128 quantisation of w [G,K,N] -> (packed codes uint8 [G, N/16, K/128, 2048],
    scales f32 [G, K/128, N/128]).  The packed order is the one gmm_fp8_fwd reads
    (include/gmm.h, gmm_quantize_rhs)."""
    lib = load_library()
    G, K, N = w.shape
    q = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 2048), dtype=torch.uint8, device=w.device)
    s = torch.empty((G, max(K // 128, 0), max(N // 128, 0)), dtype=torch.float32, device=w.device)
    _check(lib.gmm_quantize_rhs(_ptr(w), _dt(w), G, K, N, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def gmm_pack_rhs(q: torch.Tensor) -> torch.Tensor:
    """E4M3 codes [G,K,N] (uint8 or float8_e4m3fn) quantised elsewhere -> the packed
    order gmm_fp8_fwd reads, uint8 [G, N/16, K/128, 2048] (include/gmm.h, gmm_pack_rhs)."""
    lib = load_library()
    G, K, N = q.shape
    packed = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 2048), dtype=torch.uint8,
                         device=q.device)
    _check(lib.gmm_pack_rhs(_ptr(q), G, K, N, _ptr(packed), _stream(q)))
    return packed


def gmm_quant_scales(amax: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """The recipe's scale pair for block abs-maxima amax (fp32): (a/448, guarded inverse)."""
    lib = load_library()
    n = amax.numel()
    scale = torch.empty_like(amax)
    inv = torch.empty_like(amax)
    _check(lib.gmm_quant_scales(_ptr(amax), n, _ptr(scale), _ptr(inv), _stream(amax)))
    return scale, inv


def gmm_quantize_rhs_mxfp4(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP4 quantisation of w [G,K,N] -> (packed E2M1 codes uint8 [G, N/16, K/128, 1024],
    E8M0 scales uint8 [G, N/16, K/128, 64]), in the order gmm_fp8_mxfp4_fwd reads
    (include/gmm.h, gmm_quantize_rhs_mxfp4)."""
    lib = load_library()
    G, K, N = w.shape
    q = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 1024), dtype=torch.uint8, device=w.device)
    s = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 64), dtype=torch.uint8, device=w.device)
    _check(lib.gmm_quantize_rhs_mxfp4(_ptr(w), _dt(w), G, K, N, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def gmm_fp8_mxfp4_fwd(lhs: torch.Tensor, rhs_q: torch.Tensor, rhs_scale: torch.Tensor,
                      group_sizes: torch.Tensor, lhs_scale: Optional[torch.Tensor] = None,
                      out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GMM of a 1x128 FP8 LHS (bf16/fp32 quantised in-kernel, or uint8 codes with
    lhs_scale [M,K/128]) against MXFP4 weights from gmm_quantize_rhs_mxfp4."""
    lib = load_library()
    M, K = lhs.shape
    G, N16, KB, chunk = rhs_q.shape
    N = N16 * 16
    if chunk != 1024 or KB * 128 != K or tuple(rhs_scale.shape) != (G, N16, KB, 64):
        raise ValueError("rhs_q %s / rhs_scale %s do not match K=%d"
                         % (tuple(rhs_q.shape), tuple(rhs_scale.shape), K))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    ws, wsp, wsb = _ws(ws, OP_FP8_MXFP4_FWD, M, K, N, G, lhs.device)
    _check(lib.gmm_fp8_mxfp4_fwd(_ptr(lhs), _dt(lhs), _ptr(lhs_scale), _ptr(rhs_q),
                                 _ptr(rhs_scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
                                 _dt(out), wsp, wsb, _stream(lhs)))
    return out


def gmm_quantize_rhs_int4(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """int4 quantisation of w [G,K,N] -> (packed two's-complement codes uint8
    [G, N/16, K/128, 1024], scales f32 [G, K/128, N/128]), in the order
    gmm_fp8_int4_fwd reads (include/gmm.h, gmm_quantize_rhs_int4)."""
    lib = load_library()
    G, K, N = w.shape
    q = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 1024), dtype=torch.uint8, device=w.device)
    s = torch.empty((G, max(K // 128, 0), max(N // 128, 0)), dtype=torch.float32, device=w.device)
    _check(lib.gmm_quantize_rhs_int4(_ptr(w), _dt(w), G, K, N, _ptr(q), _ptr(s), _stream(w)))
    return q, s


def gmm_pack_rhs_int4(q: torch.Tensor) -> torch.Tensor:
    """int4 codes made elsewhere (int8 values in [-8, 7], [G,K,N]) -> the packed
    order gmm_fp8_int4_fwd reads, uint8 [G, N/16, K/128, 1024]."""
    lib = load_library()
    if q.dtype != torch.int8:
        raise ValueError("int4 codes are passed as int8, got %s" % q.dtype)
    G, K, N = q.shape
    packed = torch.empty((G, max(N // 16, 0), max(K // 128, 0), 1024), dtype=torch.uint8,
                         device=q.device)
    _check(lib.gmm_pack_rhs_int4(_ptr(q), G, K, N, _ptr(packed), _stream(q)))
    return packed


def gmm_fp8_int4_fwd(lhs: torch.Tensor, rhs_q: torch.Tensor, rhs_scale: torch.Tensor,
                     group_sizes: torch.Tensor, lhs_scale: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GMM of a 1x128 FP8 LHS (bf16/fp32 quantised in-kernel, or uint8 codes with
    lhs_scale [M,K/128]) against int4 weights from gmm_quantize_rhs_int4 (or
    gmm_pack_rhs_int4 with their [G,K/128,N/128] scales)."""
    lib = load_library()
    M, K = lhs.shape
    G, N16, KB, chunk = rhs_q.shape
    N = N16 * 16
    if chunk != 1024 or KB * 128 != K or tuple(rhs_scale.shape) != (G, KB, N // 128):
        raise ValueError("rhs_q %s / rhs_scale %s do not match K=%d"
                         % (tuple(rhs_q.shape), tuple(rhs_scale.shape), K))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    ws, wsp, wsb = _ws(ws, OP_FP8_INT4_FWD, M, K, N, G, lhs.device)
    _check(lib.gmm_fp8_int4_fwd(_ptr(lhs), _dt(lhs), _ptr(lhs_scale), _ptr(rhs_q),
                                _ptr(rhs_scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
                                _dt(out), wsp, wsb, _stream(lhs)))
    return out


def gmm_fp8_fwd(lhs: torch.Tensor, rhs_q: torch.Tensor, rhs_scale: torch.Tensor,
                group_sizes: torch.Tensor, lhs_scale: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                q_out: Optional[torch.Tensor] = None, scale_out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Blockwise-FP8 GMM.  lhs [M,K] bf16/fp32 (quantised in-kernel) or uint8 codes
    with lhs_scale [M,K/128]; rhs_q, rhs_scale as returned by gmm_quantize_rhs."""
    lib = load_library()
    M, K = lhs.shape
    G, N16, KB, slab = rhs_q.shape
    N = N16 * 16
    if slab != 2048 or KB * 128 != K:
        raise ValueError("rhs_q shape %s does not match K=%d" % (tuple(rhs_q.shape), K))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    ws, wsp, wsb = _ws(ws, OP_FP8_FWD, M, K, N, G, lhs.device)
    _check(lib.gmm_fp8_fwd(_ptr(lhs), _dt(lhs), _ptr(lhs_scale), _ptr(rhs_q), _ptr(rhs_scale),
                           _ptr(group_sizes), M, K, N, G, _ptr(out), _dt(out), _ptr(q_out),
                           _ptr(scale_out), wsp, wsb, _stream(lhs)))
    return out


def gmm_fp8_fwd_noalloc(lhs: torch.Tensor, rhs_q: torch.Tensor, rhs_scale: torch.Tensor,
                        group_sizes: torch.Tensor, lhs_scale: Optional[torch.Tensor] = None,
                        out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                        q_out: Optional[torch.Tensor] = None,
                        scale_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gmm_fp8_fwd without a workspace (the library's own static device scratch;
    the C call allocates nothing).  Pass `out` to keep this wrapper from
    allocating it."""
    lib = load_library()
    M, K = lhs.shape
    G, N16, KB, slab = rhs_q.shape
    N = N16 * 16
    if slab != 2048 or KB * 128 != K:
        raise ValueError("rhs_q shape %s does not match K=%d" % (tuple(rhs_q.shape), K))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    _check(lib.gmm_fp8_fwd_noalloc(_ptr(lhs), _dt(lhs), _ptr(lhs_scale), _ptr(rhs_q),
                                   _ptr(rhs_scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
                                   _dt(out), _ptr(q_out), _ptr(scale_out), _stream(lhs)))
    return out


def gmm_fp8_fwd_swiglu(lhs: torch.Tensor, rhs_q: torch.Tensor, rhs_scale: torch.Tensor,
                       group_sizes: torch.Tensor, lhs_scale: Optional[torch.Tensor] = None,
                       out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                       act_q: Optional[torch.Tensor] = None, act_scale: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused gate+up blockwise-FP8 GMM: rhs_q/rhs_scale quantise the [G,K,2N]
    concatenation (gate columns first); returns silu(gate) * up, [M,N].
    act_q [M,N] uint8 / act_scale [M,N/128] f32 optionally receive its 1x128
    quantisation."""
    lib = load_library()
    M, K = lhs.shape
    G, N16, KB, slab = rhs_q.shape
    if slab != 2048 or KB * 128 != K or N16 % 2:
        raise ValueError("rhs_q shape %s does not match K=%d" % (tuple(rhs_q.shape), K))
    N = N16 * 16 // 2
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    ws, wsp, wsb = _ws(ws, OP_FP8_FWD_SWIGLU, M, K, N, G, lhs.device)
    _check(lib.gmm_fp8_fwd_swiglu(_ptr(lhs), _dt(lhs), _ptr(lhs_scale), _ptr(rhs_q),
                                  _ptr(rhs_scale), _ptr(group_sizes), M, K, N, G, _ptr(out),
                                  _dt(out), _ptr(act_q), _ptr(act_scale), wsp, wsb, _stream(lhs)))
    return out


def gmm_bf16_fwd(lhs: torch.Tensor, rhs: torch.Tensor, group_sizes: torch.Tensor,
                 out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                 ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 GMM: out [M,N] = lhs [M,K] . rhs[g] [K,N] per group."""
    lib = load_library()
    M, K = lhs.shape
    G, K2, N = rhs.shape
    if K2 != K:
        raise ValueError("lhs K=%d but rhs K=%d" % (K, K2))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=lhs.device)
    ws, wsp, wsb = _ws(ws, OP_BF16_FWD, M, K, N, G, lhs.device)
    _check(lib.gmm_bf16_fwd(_ptr(lhs), _ptr(rhs), _ptr(group_sizes), M, K, N, G, _ptr(out),
                            _dt(out), wsp, wsb, _stream(lhs)))
    return out


def tgmm_bf16(x: torch.Tensor, dy: torch.Tensor, group_sizes: torch.Tensor,
              out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dW [G,K,N]: dW[g] = X_g^T dY_g for x [M,K], dy [M,N]."""
    lib = load_library()
    M, K = x.shape
    M2, N = dy.shape
    if M2 != M:
        raise ValueError("x has %d rows but dy has %d" % (M, M2))
    G = group_sizes.numel()
    if out is None:
        out = torch.empty((G, K, N), dtype=out_dtype, device=x.device)
    ws, wsp, wsb = _ws(ws, OP_TGMM, M, K, N, G, x.device)
    _check(lib.tgmm_bf16(_ptr(x), _ptr(dy), _ptr(group_sizes), M, K, N, G, _ptr(out), _dt(out),
                         wsp, wsb, _stream(x)))
    return out


def gmm_bf16_dx(dy: torch.Tensor, w: torch.Tensor, group_sizes: torch.Tensor,
                out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dX [M,K] = dY [M,N] . w[g]^T per group, w [G,K,N]."""
    lib = load_library()
    M, N = dy.shape
    G, K, N2 = w.shape
    if N2 != N:
        raise ValueError("dy N=%d but w N=%d" % (N, N2))
    if out is None:
        out = torch.empty((M, K), dtype=out_dtype, device=dy.device)
    ws, wsp, wsb = _ws(ws, OP_DX, M, K, N, G, dy.device)
    _check(lib.gmm_bf16_dx(_ptr(dy), _ptr(w), _ptr(group_sizes), M, K, N, G, _ptr(out),
                           _dt(out), wsp, wsb, _stream(dy)))
    return out
