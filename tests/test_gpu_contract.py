"""GPU: the boundary's contract (include/gmm.h conventions).

- Every grouped call writes its device status word into the workspace: 0 for
  group sizes that keep the contract, GMM_DEV_* bits otherwise.
- Sizes that break the contract (a negative size, sizes summing past M) never
  make a kernel touch rows outside [0, M): every buffer sits between guard rows
  that must keep their sentinel, and the result equals the oracle's result for
  the clipped groups (negative sizes read as 0, rows cut at M).
- gmm_pack_rhs: [G,K,N] E4M3 codes quantised elsewhere (by the oracle here)
  feed the forward directly.
- gmm_quant_scales: the quantisers' scale pair, bit for bit against the
  oracle over every significand of a binade of block abs-maxima and a sample
  of every exponent of the contract's range.
"""
import numpy as np
import pytest
import torch

import moe_grouped_gemm_gmm_amd as gmm
import oracle
import workloads
from helpers import assert_bf16_parity, assert_fp8_parity, to_np64, unpack_rhs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 320   # rows of sentinel before and after every row-indexed buffer


def guarded(rows, cols, dtype, fill):
    """(whole buffer, the [rows, cols] view between its guard rows)."""
    big = torch.full((GUARD + rows + GUARD, cols), fill, dtype=dtype, device=DEV)
    return big, big[GUARD:GUARD + rows]


def guarded_from(t):
    big, view = guarded(t.shape[0], t.shape[1], t.dtype, 0)
    big[:GUARD] = 1e4          # large values: any read of them would show in the result
    big[GUARD + t.shape[0]:] = -1e4
    view.copy_(t.to(DEV))
    return big, view


def clipped_sizes(gs, M):
    o = np.concatenate([[0], np.cumsum(np.maximum(gs.astype(np.int64), 0))])
    lo, hi = np.minimum(o[:-1], M), np.minimum(o[1:], M)
    return (hi - lo).astype(np.int32)


def expected_status(gs, M):
    return ((gmm.DEV_SUM_GT_M if np.maximum(gs.astype(np.int64), 0).sum() > M else 0)
            | (gmm.DEV_NEGATIVE_SIZE if (gs < 0).any() else 0))


def guards_intact(big, rows, fill_is_nan=True):
    g = torch.cat([big[:GUARD], big[GUARD + rows:]]).float()
    return bool(torch.isnan(g).all()) if fill_is_nan else True


CASES = [
    ([160, 160, 40], 256),        # sum past M: group 1 cut, group 2 empty
    ([-7, 100, 60], 256),         # a negative size
    ([0, 300, -2, 50], 256),      # both
    ([96, 64, 96], 256),          # inside the contract (status 0)
]
K, N = 256, 256


@pytest.mark.parametrize("gs,M", CASES)
def test_fp8_forwards_clip_rows(gs, M):
    gs = np.array(gs, np.int32)
    G = gs.size
    wl = workloads.custom(M, K, N, clipped_sizes(gs, M), seed=11, x_std=1.0, w_std=0.05)
    xbig, x = guarded_from(wl.x)
    gsd = torch.from_numpy(gs).to(DEV)
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8(ql, sl, qr, sr, wl.group_sizes)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    q4, e8 = gmm.gmm_quantize_rhs_mxfp4(wl.w.to(DEV))
    oq4, oe8 = oracle.quantize_rhs_mxfp4(workloads.as_f32(wl.w))
    ref4 = oracle.gmm_fp8_mxfp4(ql, sl, oq4, oe8, wl.group_sizes)
    for name, call, want in (
            ("fp8_fwd", lambda o, ws: gmm.gmm_fp8_fwd(x, rq, rs, gsd, out=o, ws=ws), ref),
            ("fp8_mxfp4_fwd", lambda o, ws: gmm.gmm_fp8_mxfp4_fwd(x, q4, e8, gsd, out=o, ws=ws), ref4)):
        obig, out = guarded(M, N, torch.float32, float("nan"))
        ws = gmm.workspace(gmm.OP_FP8_FWD, M, K, N, G, DEV)
        call(out, ws)
        torch.cuda.synchronize()
        assert guards_intact(obig, M), name
        assert gmm.device_status(ws) == expected_status(gs, M), name
        assert_fp8_parity(to_np64(out), want, name)


@pytest.mark.parametrize("gs,M", CASES)
def test_swiglu_clips_rows(gs, M):
    gs = np.array(gs, np.int32)
    wl = workloads.custom(M, K, 2 * N, clipped_sizes(gs, M), seed=12, x_std=1.0, w_std=0.05)
    xbig, x = guarded_from(wl.x)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    qr, sr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ref = oracle.gmm_fp8_swiglu(ql, sl, qr, sr, wl.group_sizes)
    obig, out = guarded(M, N, torch.float32, float("nan"))
    ws = gmm.workspace(gmm.OP_FP8_FWD_SWIGLU, M, K, N, gs.size, DEV)
    gmm.gmm_fp8_fwd_swiglu(x, rq, rs, torch.from_numpy(gs).to(DEV), out=out, ws=ws)
    torch.cuda.synchronize()
    assert guards_intact(obig, M)
    assert gmm.device_status(ws) == expected_status(gs, M)
    assert_fp8_parity(to_np64(out), ref, "swiglu")


@pytest.mark.parametrize("gs,M", CASES)
def test_bf16_calls_clip_rows(gs, M):
    gs = np.array(gs, np.int32)
    G = gs.size
    cs = clipped_sizes(gs, M)
    r = np.random.default_rng(13)
    x = torch.from_numpy(r.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(r.standard_normal((M, N), dtype=np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(r.standard_normal((G, K, N), dtype=np.float32)).to(torch.bfloat16)
    xf, dyf, wf = (workloads.as_f32(t) for t in (x, dy, w))
    _, xd = guarded_from(x)
    _, dyd = guarded_from(dy)
    wd = w.to(DEV)
    gsd = torch.from_numpy(gs).to(DEV)
    # forward and dX: row-indexed outputs between guard rows
    for name, cols, call, want in (
            ("bf16_fwd", N, lambda o, ws: gmm.gmm_bf16_fwd(xd, wd, gsd, out=o, ws=ws),
             oracle.gmm(xf, wf, cs)),
            ("dx", K, lambda o, ws: gmm.gmm_bf16_dx(dyd, wd, gsd, out=o, ws=ws),
             oracle.gmm_dx(dyf, wf, cs))):
        obig, out = guarded(M, cols, torch.float32, float("nan"))
        ws = gmm.workspace(gmm.OP_BF16_FWD, M, K, N, G, DEV)
        call(out, ws)
        torch.cuda.synchronize()
        assert guards_intact(obig, M), name
        assert gmm.device_status(ws) == expected_status(gs, M), name
        assert_bf16_parity(to_np64(out), want, name)
    # tgmm: reads x, dy rows; its dW of every group is the clipped groups' dW
    dw = torch.full((G, K, N), float("nan"), dtype=torch.float32, device=DEV)
    ws = gmm.workspace(gmm.OP_TGMM, M, K, N, G, DEV)
    gmm.tgmm_bf16(xd, dyd, gsd, out=dw, ws=ws)
    torch.cuda.synchronize()
    assert gmm.device_status(ws) == expected_status(gs, M)
    assert_bf16_parity(to_np64(dw), oracle.tgmm(xf, dyf, cs), "tgmm")


def test_status_word_is_rewritten_every_call():
    """The workspace needs no initialisation and reports the last call only."""
    M = 256
    wl = workloads.custom(M, K, N, [100, 100, 56], seed=14, x_std=1.0, w_std=0.05)
    rq, rs = gmm.gmm_quantize_rhs(wl.w.to(DEV))
    x = wl.x.to(DEV)
    ws = torch.full((gmm.workspace_bytes(gmm.OP_FP8_FWD, M, K, N, 3),), 0x7B, dtype=torch.uint8,
                    device=DEV)
    bad = torch.tensor([200, -1, 100], dtype=torch.int32, device=DEV)
    good = torch.from_numpy(wl.group_sizes).to(DEV)
    gmm.gmm_fp8_fwd(x, rq, rs, bad, ws=ws)
    assert gmm.device_status(ws) == gmm.DEV_SUM_GT_M | gmm.DEV_NEGATIVE_SIZE
    gmm.gmm_fp8_fwd(x, rq, rs, good, ws=ws)
    assert gmm.device_status(ws) == 0


# ------------------------------------------------------------ RHS pack ----

@pytest.mark.parametrize("G,K,N", [(1, 128, 128), (3, 384, 256), (32, 2048, 512)])
def test_pack_rhs_matches_quantiser_layout(G, K, N):
    r = np.random.default_rng(G * 7 + K)
    w = (r.standard_normal((G, K, N), dtype=np.float32) * np.float32(0.02))
    oq, osr = oracle.quantize_rhs(w)
    packed = gmm.gmm_pack_rhs(torch.from_numpy(oq).to(DEV))
    mine, _ = gmm.gmm_quantize_rhs(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), mine.cpu().numpy())
    assert np.array_equal(unpack_rhs(packed.cpu().numpy()), oq)


def test_forward_on_codes_quantised_elsewhere():
    """[G,K,N] codes + [G,K/128,N/128] scales from the oracle, packed by the
    library, with LHS codes from the oracle too: the forward matches the
    oracle on exactly those codes."""
    wl = workloads.make("tiny", seed=3)
    oq, osr = oracle.quantize_rhs(workloads.as_f32(wl.w))
    ql, sl = oracle.quantize_lhs(workloads.as_f32(wl.x))
    packed = gmm.gmm_pack_rhs(torch.from_numpy(oq).to(DEV))
    out = gmm.gmm_fp8_fwd(torch.from_numpy(ql).to(DEV), packed, torch.from_numpy(osr).to(DEV),
                          torch.from_numpy(wl.group_sizes).to(DEV),
                          lhs_scale=torch.from_numpy(sl).to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_fp8_parity(to_np64(out), oracle.gmm_fp8(ql, sl, oq, osr, wl.group_sizes), "packed")


# ---------------------------------------------------------- scale pair ----

def test_quant_scales_every_significand():
    """Every fp32 significand of a in [2^9, 2^10) (dividing by 448 and
    inverting commute with powers of two while s and 1/s stay normal, which
    the contract's range [2^-100, FLT_MAX] guarantees), plus the first, last
    and 4096 random significands of every exponent of that range and zero:
    scale and inverse bit for bit against the oracle's IEEE divisions."""
    binade = ((np.uint32(136) << 23) + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)
    r = np.random.default_rng(5)
    parts = [binade, np.zeros(1, np.float32)]
    for e in range(-100, 128):
        sig = np.concatenate([[0, 1, (1 << 23) - 1], r.integers(0, 1 << 23, size=4096)])
        parts.append((((e + 127) << 23) + sig).astype(np.uint32).view(np.float32))
    a = np.concatenate(parts)
    s, inv = gmm.gmm_quant_scales(torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    os_, oinv = oracle.quant_scales(a)
    s, inv = s.cpu().numpy(), inv.cpu().numpy()
    bad_s = np.flatnonzero(s.view(np.uint32) != os_.view(np.uint32))
    bad_i = np.flatnonzero(inv.view(np.uint32) != oinv.view(np.uint32))
    assert bad_s.size == 0, ("scale", a[bad_s[:5]], s[bad_s[:5]], os_[bad_s[:5]])
    assert bad_i.size == 0, ("inverse", a[bad_i[:5]], inv[bad_i[:5]], oinv[bad_i[:5]])
