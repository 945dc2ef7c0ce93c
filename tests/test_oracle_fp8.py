"""Pins of the oracle's E4M3 format and fp8 quantisation (CPU only).

Checked against torch's float8_e4m3fn cast (an independent library route),
hand values of the format, and properties that a slip in exponent bias,
subnormal handling, rounding direction or scale would break."""
import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_hand_values():
    cases = {1.0: 0x38, -1.0: 0xB8, 0.1: 0x1D, 448.0: 0x7E, -448.0: 0xFE, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08,
             1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 240.0: 0x77, 232.0: 0x76,
             248.0: 0x78, 0.0: 0x00}
    for x, c in cases.items():
        assert int(fp8.e4m3_encode(np.float32(x))) == c, (x, hex(int(fp8.e4m3_encode(np.float32(x)))), hex(c))


def test_matches_torch_cast():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(50000) * 60, g.standard_normal(20000) * 0.01,
                        g.uniform(-448, 448, 20000)]).astype(np.float32).clip(-448, 448)
    assert np.array_equal(fp8.e4m3_encode(x), _torch_codes(x))


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = fp8.e4m3_decode(codes)
    back = fp8.e4m3_encode(vals.astype(np.float32))
    nz = vals != 0
    assert np.array_equal(back[nz], codes[nz])
    assert np.isnan(fp8.e4m3_decode(np.uint8(0x7F))) and np.nanmax(vals) == 448.0
    # the finite values, sorted, are strictly increasing (monotone code order per sign)
    pos = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_nearest_and_ties_to_even():
    g = np.random.default_rng(1)
    x = g.uniform(-448, 448, 20000).astype(np.float32)
    q = fp8.e4m3_decode(fp8.e4m3_encode(x))
    grid = np.unique(np.abs(fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    grid = np.concatenate([-grid[::-1], grid])
    nearest = np.min(np.abs(grid[None, :] - x[:, None].astype(np.float64)), axis=1)
    assert np.all(np.abs(q - x) <= nearest + 0.0)
    # relative error at most half a unit: 2^-4 for normal values
    n = np.abs(x) >= 2.0 ** -6
    assert np.max(np.abs(q[n] - x[n]) / np.abs(x[n])) <= 2.0 ** -4


def test_per_head_scale_maps_amax_to_448():
    g = np.random.default_rng(2)
    x = (g.standard_normal((300, 3, 64)) * np.array([0.5, 3.0, 40.0])[None, :, None]).astype(np.float32)
    codes, s = fp8.quantize_per_head(x)
    assert s.dtype == np.float32 and s.shape == (3,)
    for h in range(3):
        assert s[h] == np.float32(np.max(np.abs(x[:, h])) / np.float32(448.0))
        assert np.max(fp8.e4m3_decode(codes[:, h]) * 1.0) == pytest.approx(448.0) or \
            np.min(fp8.e4m3_decode(codes[:, h])) == pytest.approx(-448.0)
    deq = fp8.dequantize(codes, s[None, :, None])
    rel = np.abs(deq - x) / np.maximum(np.abs(x), 2.0 ** -6 * s[None, :, None])
    assert np.max(rel) <= 2.0 ** -4 + 1e-12
    assert np.array_equal(fp8.absmax_scale(np.zeros(4)), np.float32(1.0))


def test_w8a8_matmul_exact_and_bounded():
    g = np.random.default_rng(3)
    # values on the fp8 grid with amax exactly 448 per row / column: quantisation is exact
    grid = fp8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    a = g.choice(grid, size=(20, 32)) * g.choice([-1, 1], size=(20, 32))
    a[:, 0] = 448.0
    w = g.choice(grid, size=(32, 16)) * g.choice([-1, 1], size=(32, 16))
    w[0, :] = 448.0
    assert np.array_equal(fp8.w8a8_matmul(a, w), a.astype(np.float64) @ w)
    # general inputs: within the bound set by one half-unit rounding of each factor
    a = g.standard_normal((64, 96)).astype(np.float32)
    w = (g.standard_normal((96, 48)) * 0.1).astype(np.float32)
    y = fp8.w8a8_matmul(a, w)
    ref = a.astype(np.float64) @ w
    sa = fp8.absmax_scale(a, axis=1)[:, None] * 2.0 ** -9
    sw = fp8.absmax_scale(w, axis=0)[None, :] * 2.0 ** -9
    bound = (np.abs(a) * 2.0 ** -4 + sa) @ np.abs(w) + np.abs(a) @ (np.abs(w) * 2.0 ** -4 + sw) \
        + (np.abs(a) * 2.0 ** -4 + sa) @ (np.abs(w) * 2.0 ** -4 + sw)
    assert np.all(np.abs(y - ref) <= bound)
    # per-row scales: a power-of-two row factor scales that row of y exactly
    a2 = a.copy()
    a2[5] *= 8.0
    y2 = fp8.w8a8_matmul(a2, w)
    assert np.array_equal(y2[5], 8.0 * y[5]) and np.array_equal(np.delete(y2, 5, 0), np.delete(y, 5, 0))
