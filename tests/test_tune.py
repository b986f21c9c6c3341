"""The tile search's host logic (no GPU): the configuration space of every
phase, which configurations fit which shapes (asked of the library's own
resolver, which runs on the host), the staged gate, and the library's
default choices at the benchmark's shapes."""
import numpy as np
import pytest

import moe_grouped_gemm_gmm_amd as gmm
from moe_grouped_gemm_gmm_amd import tune


def test_space_and_names():
    for phase in tune.PHASES:
        sp = tune.space(phase)
        assert sp[0] == {}
        names = [tune.config_name(c) for c in sp]
        assert len(set(names)) == len(names) and names[0] == "default"
    fp8 = tune.space("fp8_fwd")
    assert {c.get("kernel") for c in fp8[1:]} == {1, 2, 3}
    assert {c["waves"] for c in fp8 if c.get("kernel") == 1} == {8, 12, 16}
    assert {c.get("placement") for c in fp8 if c.get("kernel") == 1} == {None, 2}
    assert {(c["tile_m"], c["tile_n"]) for c in fp8 if c.get("kernel") == 2} == {
        (m, n) for m in (48, 64) for n in (128, 256, 512)}
    assert [c.get("placement") for c in tune.space("tgmm")] == [None, 1, 2, 1, 2, 1, 2] + [1, 2] * 8
    assert [c.get("placement") for c in tune.space("dx")] == [None, 1, 2, 1, 2, None] + [1, 2] * 8
    assert [c.get("waves") for c in tune.space("bf16_fwd") if c.get("kernel") == 3].count(8) == 4
    assert {c.get("kernel") for c in tune.space("dx")} == {None, 2, 3}
    assert {(c["depth"], c["residency"]) for c in tune.space("bf16_fwd")
            if c.get("kernel") == 3 and "depth" in c} == set(tune.DMA_PAIRS)
    with pytest.raises(ValueError):
        tune.space("nope")


def test_candidates_follow_the_shape():
    wi = tune.candidates("fp8_fwd", (8192, 2048, 512, 32))
    names = {tune.config_name(c) for c in wi}
    assert "kernel=1,waves=16" in names and "kernel=3,tile_n=256" in names
    assert "kernel=3,tile_n=512" not in names          # 512-column row-resident tiles need K <= 1024
    n384 = {tune.config_name(c) for c in tune.candidates("fp8_fwd", (1024, 256, 384, 4))}
    assert not any(n.startswith("kernel=1") for n in n384)   # warp-specialised needs N % 512 == 0
    assert "kernel=2,tile_m=48,tile_n=128" in n384 and "kernel=2,tile_m=48,tile_n=256" not in n384
    mx = {tune.config_name(c) for c in tune.candidates("mxfp4_fwd", (8192, 512, 2048, 32))}
    assert "kernel=3" in mx and "kernel=1,tile_n=512" in mx
    tg = {tune.config_name(c) for c in tune.candidates("tgmm", (700, 256, 256, 6))}
    assert "placement=2,residency=3" not in tg         # 4 tiles per group cannot spread over 8 XCDs
    assert "kernel=2,placement=1" in tg and "kernel=2,placement=2" not in tg
    dx = {tune.config_name(c) for c in tune.candidates("dx", (700, 384, 256, 6))}
    assert "kernel=2" not in dx                        # 256 x 256 tiles need K % 256 == 0
    assert "placement=1,residency=2" in tg
    assert "depth=3,kernel=3,placement=1,residency=3" in tg
    assert "depth=3,kernel=3,placement=2,residency=3" not in tg
    assert {"depth=%d,kernel=3,placement=%d,residency=%d" % (d, p, r)
            for d, r in tune.DMA_PAIRS for p in (1, 2)} <= dx
    assert "kernel=3,placement=1,waves=8" in dx
    assert "kernel=3,placement=1,tile_n=256,waves=8" not in dx          # 128 x 256 dX tiles need K % 256 == 0
    dx512 = {tune.config_name(c) for c in tune.candidates("dx", (700, 512, 256, 6))}
    assert "kernel=3,placement=1,tile_n=256,waves=8" in dx512
    assert "kernel=3,placement=1,waves=8" in tg
    tg384 = {tune.config_name(c) for c in tune.candidates("tgmm", (700, 384, 256, 6))}
    assert "kernel=3,placement=1,waves=8" not in tg384   # 8-wave tgmm tiles need K % 256 == 0


def test_bf16_load_to_lds_kernel_config():
    """kernel 3: depth = LDS stages, residency = workgroups per CU, in the
    pairs the LDS holds (2 x 2, 3 x 1-3, 4 x 1-2; default 3 x 3); depth is
    rejected on the other bf16 kernels."""
    B, T = gmm.OP_BF16_FWD, gmm.OP_TGMM
    nz = lambda d: {k: v for k, v in d.items() if v}
    try:
        gmm.set_tile_config(B, {"kernel": 3})
        assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32)) == {
            "kernel": 3, "waves": 4, "depth": 3, "residency": 3, "placement": 1}
        # kernel 3 keeps row tiles aligned to absolute rows at any grid size
        # (production shape forward 265 us against 282 with group-start tiles)
        assert nz(gmm.get_tile_config(B, 65536, 2048, 512, 256))["placement"] == 1
        for d, r in tune.DMA_PAIRS:
            gmm.set_tile_config(B, {"kernel": 3, "depth": d, "residency": r})
            assert gmm.get_tile_config(B, 8192, 2048, 512, 32)["residency"] == r
        gmm.set_tile_config(B, {"kernel": 3, "depth": 2})
        assert gmm.get_tile_config(B, 8192, 2048, 512, 32)["residency"] == 2
        gmm.set_tile_config(B, {"kernel": 3, "depth": 4})
        assert gmm.get_tile_config(B, 8192, 2048, 512, 32)["residency"] == 2
        for bad in ({"kernel": 3, "depth": 5}, {"kernel": 3, "depth": 1}, {"kernel": 3, "depth": 2, "residency": 3},
                    {"kernel": 3, "depth": 4, "residency": 3}, {"kernel": 3, "depth": 2, "residency": 1},
                    {"kernel": 1, "depth": 2}, {"kernel": 2, "depth": 2}, {"kernel": 4}):
            with pytest.raises(gmm.GmmError):
                gmm.set_tile_config(B, bad)
                gmm.get_tile_config(B, 8192, 2048, 512, 32)
        gmm.set_tile_config(B, {"depth": 2})              # depth alone: kernel 3
        assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32))["kernel"] == 3
        gmm.set_tile_config(B, {"residency": 2})          # residency alone: kernel 1
        assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32)) == {"kernel": 1, "residency": 2, "placement": 1}
        gmm.set_tile_config(T, {"kernel": 3, "depth": 3, "placement": 2})
        assert nz(gmm.get_tile_config(T, 8192, 2048, 512, 32)) == {
            "kernel": 3, "waves": 4, "depth": 3, "residency": 3, "placement": 2}
        # 8 waves: 256 x 128 tiles, 3 stages, two workgroups per CU
        gmm.set_tile_config(B, {"kernel": 3, "waves": 8})
        assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32)) == {
            "kernel": 3, "waves": 8, "tile_n": 128, "depth": 3, "residency": 2, "placement": 1}
        gmm.set_tile_config(T, {"kernel": 3, "waves": 8})
        assert gmm.get_tile_config(T, 8192, 2048, 512, 32)["waves"] == 8
        with pytest.raises(gmm.GmmError):
            gmm.get_tile_config(T, 8192, 384, 512, 32)       # K not a multiple of 256
        gmm.set_tile_config(T, {"kernel": 3, "waves": 8, "placement": 2})
        with pytest.raises(gmm.GmmError):                    # 2 x 2 tiles per group cannot spread over 8 XCDs
            gmm.get_tile_config(T, 8192, 512, 256, 32)
        assert gmm.get_tile_config(T, 8192, 2048, 512, 32)["placement"] == 2
        gmm.set_tile_config(B, {"kernel": 3, "waves": 8, "tile_n": 256})     # 128 x 256 tiles
        assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32)) == {
            "kernel": 3, "waves": 8, "tile_n": 256, "depth": 3, "residency": 2, "placement": 1}
        with pytest.raises(gmm.GmmError):
            gmm.get_tile_config(B, 8192, 2048, 384, 32)      # N not a multiple of 256
        for bad in ({"kernel": 3, "waves": 8, "depth": 2}, {"kernel": 3, "waves": 8, "residency": 3},
                    {"kernel": 3, "waves": 6}, {"kernel": 1, "waves": 8}, {"waves": 4},
                    {"kernel": 3, "tile_n": 256}, {"kernel": 3, "waves": 4, "tile_n": 256},
                    {"kernel": 3, "waves": 8, "tile_n": 512}, {"kernel": 3, "waves": 8, "tile_m": 128}):
            with pytest.raises(gmm.GmmError):
                gmm.set_tile_config(B, bad)
                gmm.get_tile_config(B, 8192, 2048, 512, 32)
        with pytest.raises(gmm.GmmError):                    # the FP8 forward has no 4-wave form
            gmm.set_tile_config(gmm.OP_FP8_FWD, {"kernel": 1, "waves": 4})
            gmm.get_tile_config(gmm.OP_FP8_FWD, 8192, 2048, 512, 32)
    finally:
        gmm.set_tile_config(B, None)
        gmm.set_tile_config(T, None)
        gmm.set_tile_config(gmm.OP_FP8_FWD, None)


def test_library_default_choices():
    """The library's own choice at the benchmark's shapes (the host resolver;
    with no GPU the CU count is taken as 256, the MI355X's)."""
    F, S, X, B, T, D = (gmm.OP_FP8_FWD, gmm.OP_FP8_FWD_SWIGLU, gmm.OP_FP8_MXFP4_FWD,
                        gmm.OP_BF16_FWD, gmm.OP_TGMM, gmm.OP_DX)
    nz = lambda d: {k: v for k, v in d.items() if v}
    assert nz(gmm.get_tile_config(F, 8192, 2048, 512, 32)) == {
        "kernel": 1, "waves": 16, "tile_m": 48, "tile_n": 512, "depth": 1, "placement": 2}
    assert gmm.get_tile_config(F, 8192, 2048, 512, 32, lhs_dtype=gmm.GMM_E4M3)["placement"] == 1
    assert gmm.get_tile_config(F, 4096, 2048, 512, 100)["placement"] == 1   # G beyond one scan chunk
    assert nz(gmm.get_tile_config(F, 8192, 512, 2048, 32)) == {"kernel": 3, "tile_m": 48, "tile_n": 512}
    assert nz(gmm.get_tile_config(F, 65536, 2048, 512, 256)) == {"kernel": 2, "tile_m": 64, "tile_n": 512}
    assert nz(gmm.get_tile_config(S, 8192, 2048, 512, 32)) == {"kernel": 2, "tile_m": 48, "tile_n": 256}
    assert nz(gmm.get_tile_config(X, 8192, 2048, 512, 32))["kernel"] == 1
    # bf16: the load-to-LDS kernel (3 stages x 3 workgroups per CU) for forward / dX
    # grids of at most 8 workgroups per CU
    dma = {"kernel": 3, "waves": 4, "depth": 3, "residency": 3}
    assert nz(gmm.get_tile_config(B, 8192, 2048, 512, 32)) == dict(dma, placement=1)
    # tgmm: the 8-wave 256 x 128 tiles for 128 or more groups when K is a multiple of 256
    dma8 = {"kernel": 3, "waves": 8, "tile_n": 128, "depth": 3, "residency": 2}
    assert nz(gmm.get_tile_config(T, 65536, 2048, 512, 256)) == dma8
    assert nz(gmm.get_tile_config(T, 65536, 2048, 512, 128)) == dma8
    assert nz(gmm.get_tile_config(T, 8192, 2048, 512, 32)) == dma
    assert nz(gmm.get_tile_config(T, 65536, 384, 512, 256)) == dma
    assert nz(gmm.get_tile_config(D, 8192, 2048, 512, 32)) == dict(dma, placement=2)   # dX: group-start rows
    # larger forward / dX grids: the 8-wave 128 x 256 tiles, row tiles from each group's start
    wide = {"kernel": 3, "waves": 8, "tile_n": 256, "depth": 3, "residency": 2, "placement": 2}
    assert nz(gmm.get_tile_config(D, 65536, 2048, 512, 256)) == wide
    assert nz(gmm.get_tile_config(B, 65536, 2048, 512, 256)) == wide
    # ... and kernel 1 where the tiled columns are not a multiple of 256
    assert nz(gmm.get_tile_config(B, 65536, 2048, 384, 256)) == {"kernel": 1, "residency": 3, "placement": 2}
    assert all(v in (1, 2, 3, 4) for v in gmm.get_tile_config(D, 8192, 2048, 512, 32).values() if v)


def test_set_tile_config_checks_fields_and_fit():
    F = gmm.OP_FP8_FWD
    try:
        with pytest.raises(gmm.GmmError):
            gmm.set_tile_config(F, {"waves": 10})
        with pytest.raises(ValueError):
            gmm.set_tile_config(F, {"wavez": 16})
        gmm.set_tile_config(F, {"kernel": 1, "waves": 16, "depth": 2})
        with pytest.raises(gmm.GmmError):        # two steps of weights need 12 waves
            gmm.get_tile_config(F, 8192, 2048, 512, 32)
        gmm.set_tile_config(F, {"kernel": 2, "tile_n": 256, "tile_m": 64})
        assert gmm.get_tile_config(F, 8192, 2048, 512, 32)["tile_n"] == 256
    finally:
        gmm.set_tile_config(F, None)
    assert gmm.get_tile_config(F, 8192, 2048, 512, 32)["waves"] == 16


def test_gate_bars():
    ref = np.linspace(-2.0, 2.0, 1001)
    assert tune.gate(ref.copy(), ref, tune.STRICT)["pass"]
    edge = ref + 0.999 * (1e-3 + 1e-2 * np.abs(ref))            # inside the strict bar
    assert tune.gate(edge, ref, tune.STRICT)["excess"] <= 0
    noisy = ref + 0.02
    assert not tune.gate(noisy, ref, tune.STRICT)["pass"]       # beyond atol 1e-3
    assert tune.gate(noisy, ref, tune.RELAXED)["pass"]          # within atol 1e-1, SNR > 20 dB
    far = ref * 0.5
    g = tune.gate(far, ref, tune.RELAXED)
    assert not g["pass"] and g["snr_db"] == pytest.approx(10 * np.log10(4.0))
    assert tune.gate(np.where(ref > 0, np.nan, ref), ref, tune.RELAXED)["excess"] == float("inf")
    assert tune.gate(np.zeros(3), ref, tune.STRICT)["pass"] is False


def test_group_sizes_routings():
    u = tune.group_sizes(8192, 32, 0, "uniform")
    z = tune.group_sizes(8192, 32, 0, "zipf")
    assert u.sum() == z.sum() == 8192 and u.dtype == z.dtype == np.int32
    assert z.max() > 4 * 8192 / 32 > u.max()
