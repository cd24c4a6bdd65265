"""Pins of the FP8 oracle (oracle/swin_fp8.py) against the E4M3 format's own
definition: landmark values, exhaustive code round trips, ties to even,
saturation, and exactness on values already on the grid."""
import numpy as np

from oracle import swin_fp8 as f8


def test_landmarks():
    dec = f8.e4m3_decode
    assert dec(0x7E) == 448.0                 # largest finite: 1.75 * 2^8
    assert dec(0x08) == 2.0 ** -6             # smallest normal
    assert dec(0x01) == 2.0 ** -9             # smallest subnormal
    assert dec(0x07) == 7 * 2.0 ** -9         # largest subnormal
    assert dec(0x38) == 1.0                   # exponent field 7 = bias
    assert dec(0x3F) == 1.875
    assert dec(0xB8) == -1.0
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    assert dec(0x00) == 0.0 and dec(0x80) == 0.0


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = f8.e4m3_decode(codes)
    back = f8.e4m3_encode(vals)
    # +0 / -0 both decode to 0; the encoder keeps the sign of a negative input only.
    np.testing.assert_array_equal(back[codes != 0x80], codes[codes != 0x80])
    assert f8.e4m3_encode(np.array([-0.0]))[0] == 0x00


def test_ties_to_even_and_saturation():
    enc, dec = f8.e4m3_encode, f8.e4m3_decode
    # Between 1 and 1.125 (mantissa 0 and 1): the midpoint goes to 1 (even).
    assert dec(enc(1.0625)) == 1.0
    # Between 1.125 and 1.25 (mantissa 1 and 2): the midpoint goes to 1.25.
    assert dec(enc(1.1875)) == 1.25
    # Subnormal midpoints: 0.5 * 2^-9 -> 0, 1.5 * 2^-9 -> 2 * 2^-9.
    assert dec(enc(0.5 * 2.0 ** -9)) == 0.0
    assert dec(enc(1.5 * 2.0 ** -9)) == 2 * 2.0 ** -9
    # 7.5 * 2^-9 lies between the largest subnormal and 2^-6: ties to 8 * 2^-9.
    assert dec(enc(7.5 * 2.0 ** -9)) == 2.0 ** -6
    # Carry into the next binade: 1.9375 (between 1.875 and 2) -> 2.
    assert dec(enc(1.9375)) == 2.0
    # Saturation and sign.
    assert dec(enc(1e6)) == 448.0 and dec(enc(-1e6)) == -448.0
    assert dec(enc(464.0)) == 448.0
    assert enc(-1e-9)[()] == 0x80


def test_encode_is_nearest():
    # Brute force: every value's code is the nearest grid point (ties excluded).
    grid = f8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(0, 448, 2000), 2.0 ** rng.uniform(-12, 8, 2000)])
    got = f8.e4m3_decode(f8.e4m3_encode(v))
    d = np.abs(grid[None, :] - v[:, None])
    best = grid[np.argmin(d, axis=1)]
    np.testing.assert_array_equal(got, best)


def test_quantize_rows_scale_and_grid_exactness():
    rng = np.random.default_rng(5)
    # Rows already on the grid times a power-of-two scale with amax = 448 * scale:
    # quantisation is lossless, so the linear layer equals the float64 product.
    codes = rng.integers(0, 0x7E, (6, 64)).astype(np.uint8)
    codes[:, 0] = 0x7E                                   # amax hits 448 in every row
    scales = 2.0 ** rng.integers(-6, 3, 6)
    x = (f8.e4m3_decode(codes) * scales[:, None]).astype(np.float32)
    q, s = f8.quantize_rows(x)
    np.testing.assert_array_equal(f8.e4m3_decode(q), f8.e4m3_decode(codes))
    np.testing.assert_array_equal(s, scales.astype(np.float32))
    w = (f8.e4m3_decode(rng.integers(0, 0x7E, (5, 64)).astype(np.uint8)) * 0.25).astype(np.float32)
    w[:, 0] = 448 * 0.25
    qw, sw = f8.quantize_rows(w)
    b = rng.normal(size=5)
    np.testing.assert_allclose(f8.linear_fp8(q, s, qw, sw, b),
                               x.astype(np.float64) @ w.astype(np.float64).T + b, rtol=1e-12)
    # A zero row: scale 1, all codes 0.
    q0, s0 = f8.quantize_rows(np.zeros((1, 8), np.float32))
    assert s0[0] == 1.0 and not q0.any()
    # Every code's magnitude is within the clamp and the error within half a step.
    xr = rng.normal(size=(4, 256)).astype(np.float32)
    qr, sr = f8.quantize_rows(xr)
    err = np.abs(f8.e4m3_decode(qr) * sr[:, None] - xr)
    assert np.all(err <= np.abs(xr) * 2.0 ** -4 + sr[:, None] * 2.0 ** -10)
