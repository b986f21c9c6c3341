"""Pins of the oracle's E4M3 codec against torch's float8_e4m3fn (CPU).

The codec reading (OCP E4M3, round to nearest even, sign of zero kept,
finite values past 464 saturated) is the one listed with the oracle.  torch's
cast is an independent implementation of the same OCP format; it agrees with
the oracle everywhere within +-464 and returns NaN past 464, where the
oracle saturates (checked against the closed form instead).
"""
import numpy as np
import pytest
import torch

import oracle


def torch_encode(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.isnan(ours[nan]).all()
    assert np.array_equal(ours[~nan], ref[~nan])
    # closed-form anchors
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0


def _grid():
    vals = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, ascending
    assert np.all(np.diff(vals) > 0)
    return vals


def _around(points: np.ndarray, steps: int = 3) -> np.ndarray:
    p = points.astype(np.float32)
    out = [p]
    up, dn = p.copy(), p.copy()
    for _ in range(steps):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        out += [up, dn]
    return np.concatenate(out)


def test_encode_rounding_boundaries_match_torch():
    v = _grid()
    mids = (v[:-1] + v[1:]) / 2.0          # exact in fp32
    pts = _around(np.concatenate([v, mids, [448.0, 456.0, 464.0]]))
    pts = pts[np.abs(pts) <= 464.0]
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(oracle.e4m3_encode(pts), torch_encode(pts))


def test_encode_random_values_match_torch():
    r = np.random.default_rng(1234)
    mag = np.exp2(r.uniform(-14.0, np.log2(464.0), size=1_000_000)).astype(np.float32)
    sign = np.where(r.random(mag.size) < 0.5, -1.0, 1.0).astype(np.float32)
    x = mag * sign
    bits = r.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits) & (np.abs(bits) <= 464.0)]
    x = np.concatenate([x, bits])
    assert np.array_equal(oracle.e4m3_encode(x), torch_encode(x))


def test_encode_zero_sign_and_tiny():
    x = np.array([0.0, -0.0, 1e-45, -1e-45, 2.0 ** -10, -(2.0 ** -10),
                  2.0 ** -10 * 1.0001, -1e-9], dtype=np.float32)
    assert oracle.e4m3_encode(x).tolist() == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01, 0x80]


def test_encode_saturates_past_464():
    x = np.array([464.0001, 480.0, 1e6, 3.0e38, -500.0, -3.0e38], dtype=np.float32)
    assert oracle.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


@pytest.mark.parametrize("code", range(0, 0x7F))
def test_encode_decode_roundtrip(code):
    v = oracle.e4m3_decode(np.array([code], np.uint8))
    assert oracle.e4m3_encode(v.astype(np.float32))[0] == code
    assert oracle.e4m3_encode(-v.astype(np.float32))[0] == (code | 0x80)
