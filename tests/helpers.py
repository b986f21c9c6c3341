"""Shared comparison helpers for the parity tests."""
import numpy as np
import torch

# FP8 forward vs the fp64 oracle on the same codes ("GEMM Kernel 性能优化十问",
# Q9: kernel vs CPU reference of the same quantised computation).
FP8_ATOL, FP8_RTOL, FP8_MIN_SQNR_DB = 1e-3, 1e-2, 40.0
# bf16 paths: |gpu - ref| <= 1e-3 + 2e-2 |ref| (fp32 accumulation, bf16 output).
BF16_ATOL, BF16_RTOL = 1e-3, 2e-2


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def sqnr_db(ref: np.ndarray, out: np.ndarray) -> float:
    noise = np.sum((ref - out) ** 2)
    sig = np.sum(ref ** 2)
    if noise == 0:
        return float("inf")
    return float(10.0 * np.log10(sig / noise))


def assert_close(out: np.ndarray, ref: np.ndarray, atol: float, rtol: float, what: str = ""):
    err = np.abs(out - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements out of tolerance; first %s: out=%s ref=%s" % (
            what, int(bad.sum()), bad.size, idx.tolist(),
            [out[tuple(i)] for i in idx], [ref[tuple(i)] for i in idx]))


def assert_fp8_parity(out: np.ndarray, ref: np.ndarray, what: str = ""):
    assert_close(out, ref, FP8_ATOL, FP8_RTOL, what)
    if np.any(ref != 0):
        s = sqnr_db(ref, out)
        assert s > FP8_MIN_SQNR_DB, "%s: SQNR %.1f dB" % (what, s)


def assert_fp8_parity_scaled(out: np.ndarray, ref: np.ndarray, what: str = ""):
    """The FP8 bar for inputs of any scale: atol grows with the output's RMS
    (the bar above is stated for outputs of order one; the MFMA's block sums
    carry an error relative to the block's largest product, so the absolute
    error scales with the data)."""
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    # the worst excess over the unscaled bar, reported so the effect of the
    # scaling stays visible (<= 0: the unscaled bar holds as well)
    unscaled = float(np.max(np.abs(out - ref) - (FP8_ATOL + FP8_RTOL * np.abs(ref)), initial=-np.inf))
    print("%s: rms(ref) %.3g, worst excess over the unscaled bar %.3g" % (what, rms, unscaled))
    assert_close(out, ref, FP8_ATOL * max(1.0, rms), FP8_RTOL, what)
    if np.any(ref != 0):
        s = sqnr_db(ref, out)
        assert s > FP8_MIN_SQNR_DB, "%s: SQNR %.1f dB" % (what, s)
    return unscaled


def assert_bf16_parity(out: np.ndarray, ref: np.ndarray, what: str = ""):
    assert_close(out, ref, BF16_ATOL, BF16_RTOL, what)


def sample_rows_problem(group_sizes: np.ndarray, rows: np.ndarray):
    """For sorted absolute row indices, the group sizes of the sub-problem made
    of just those rows (rows keep their group)."""
    off = np.concatenate([[0], np.cumsum(group_sizes)])
    gid = np.searchsorted(off, rows, side="right") - 1
    G = group_sizes.size
    gid = np.minimum(gid, G)            # rows past the total -> tail
    sub = np.bincount(gid[gid < G], minlength=G).astype(np.int32)
    return sub, gid


def unpack_rhs(qp: np.ndarray) -> np.ndarray:
    """Packed RHS codes [G, N/16, K/128, 2048] (gmm_quantize_rhs order) -> [G, K, N]."""
    G, N16, KB, _ = qp.shape
    a = qp.reshape(G, N16, KB, 2, 4, 16, 16)          # g, nb16, kb, h, lc, lr, e
    return np.ascontiguousarray(a.transpose(0, 2, 4, 3, 6, 1, 5)).reshape(G, KB * 128, N16 * 16)


def pack_rhs(q: np.ndarray) -> np.ndarray:
    """Inverse of unpack_rhs: codes [G, K, N] -> packed [G, N/16, K/128, 2048]."""
    G, K, N = q.shape
    a = q.reshape(G, K // 128, 4, 2, 16, N // 16, 16)  # g, kb, lc, h, e, nb16, lr
    return np.ascontiguousarray(a.transpose(0, 5, 1, 3, 2, 6, 4)).reshape(G, N // 16, K // 128, 2048)


# Lane group q of the MXFP4 operand holds MX block swap2(q) of its 128-K step.
_SWAP2 = np.array([0, 2, 1, 3])


def unpack_mxfp4(qp: np.ndarray, sp: np.ndarray):
    """Packed MXFP4 weights (include/gmm.h, gmm_quantize_rhs_mxfp4) ->
    (codes [G, K, N] one per byte, E8M0 [G, K/32, N]).
    qp: [G, N/16, K/128, 1024]; sp: [G, N/16, K/128, 64]."""
    G, N16, KB, _ = qp.shape
    b = qp.reshape(G, N16, KB, 4, 16, 16)                       # lane group q, column lr, byte
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(G, N16, KB, 4, 16, 32)   # j = 2*byte + hi
    blocks = np.empty_like(nib)
    blocks[:, :, :, _SWAP2] = nib                                # index by MX block instead of q
    codes = blocks.transpose(0, 2, 3, 5, 1, 4).reshape(G, KB * 128, N16 * 16)
    s = sp.reshape(G, N16, KB, 4, 16)
    sb = np.empty_like(s)
    sb[:, :, :, _SWAP2] = s
    e8 = sb.transpose(0, 2, 3, 1, 4).reshape(G, KB * 4, N16 * 16)
    return codes, e8


def pack_mxfp4(codes: np.ndarray, e8: np.ndarray):
    """Inverse of unpack_mxfp4."""
    G, K, N = codes.shape
    KB, N16 = K // 128, N // 16
    blocks = codes.reshape(G, KB, 4, 32, N16, 16).transpose(0, 4, 1, 2, 5, 3)   # g nb kb blk lr j
    lanes = blocks[:, :, :, _SWAP2]                                             # by lane group q
    pairs = lanes.reshape(G, N16, KB, 4, 16, 16, 2)
    qp = (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8).reshape(G, N16, KB, 1024)
    s = e8.reshape(G, KB, 4, N16, 16).transpose(0, 3, 1, 2, 4)[:, :, :, _SWAP2]
    return qp, np.ascontiguousarray(s).reshape(G, N16, KB, 64).astype(np.uint8)


def unpack_int4(qp: np.ndarray) -> np.ndarray:
    """Packed int4 weights (include/gmm.h, gmm_quantize_rhs_int4) -> codes
    [G, K, N] int8.  qp: [G, N/16, K/128, 1024]; lane l of a slab holds
    column l % 16 and rows 32*(l/16) + j, byte 4d + i carrying j = 8d + i in
    its low nibble and j = 8d + 4 + i in its high one."""
    G, N16, KB, _ = qp.shape
    b = qp.reshape(G, N16, KB, 4, 16, 4, 4)                   # lane group, column, d, i
    nib = np.stack([b & 15, b >> 4], axis=-2)                  # ..., d, half, i -> j = 8d + 4 half + i
    v = ((nib.astype(np.int16) ^ 8) - 8).astype(np.int8).reshape(G, N16, KB, 4, 16, 32)
    return np.ascontiguousarray(v.transpose(0, 2, 3, 5, 1, 4)).reshape(G, KB * 128, N16 * 16)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Inverse of unpack_int4 (codes in [-8, 7])."""
    G, K, N = codes.shape
    KB, N16 = K // 128, N // 16
    v = (codes.astype(np.int16) & 15).astype(np.uint8)
    lanes = v.reshape(G, KB, 4, 32, N16, 16).transpose(0, 4, 1, 2, 5, 3)      # g nb kb lc lr j
    parts = lanes.reshape(G, N16, KB, 4, 16, 4, 2, 4)                          # j = 8d + 4 half + i
    byte = parts[..., 0, :] | (parts[..., 1, :] << 4)
    return np.ascontiguousarray(byte).reshape(G, N16, KB, 1024).astype(np.uint8)


class tile_config:
    """Context manager: a tile configuration override for one op, restored
    to the library's choice on exit (cfg None or {} keeps the default)."""

    def __init__(self, op: int, cfg):
        self.op, self.cfg = op, cfg

    def __enter__(self):
        import moe_grouped_gemm_gmm_amd as gmm
        gmm.set_tile_config(self.op, self.cfg or None)
        return self

    def __exit__(self, *exc):
        import moe_grouped_gemm_gmm_amd as gmm
        gmm.set_tile_config(self.op, None)
        return False
