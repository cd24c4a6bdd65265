"""CPU oracle for the FP8 (E4M3) linear layers of the QKV and projection GEMMs.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and imports nothing from it.

"Boosting Swin Transformer Speed", Inference Optimization: the QKV and projection
GEMMs run in 8-bit integers through cuBLASLt with per-channel scales.  The
MI355X counterpart is its native 8-bit float.  Readings (the pages fix neither
the format nor the scaling):
  * Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; normals 2^-6 .. 448, subnormals k * 2^-9; no infinities.
  * Rounding: to nearest, ties to even, after clamping to +-448 (saturation).
  * Scales: one per row of each operand: the activation per token, the weight
    per output channel.  amax = max |row| (float32), scale = amax / 448 and
    inv = 448 / amax (each one float32 division; 1 and 1 when amax = 0), code
    = E4M3(x * inv) with the product in float32.  Both sides take these
    decisions in float32, so the codes are compared bit for bit.
  * The sign bit is set exactly when x * inv < 0 (a negative value that rounds
    to zero encodes as 0x80).
  * y = (qa qw^T) * scale_a[:, None] * scale_w[None, :] + bias, the dot products
    exact (float64 here), the scaling in float64.

Parity pins (``tests/test_oracle_fp8.py``): every finite E4M3 code decodes and
re-encodes to itself; the format's landmarks (448, 2^-6, 2^-9, 1.875, ...);
ties to even on both sides of the subnormal / normal boundary; saturation;
quantisation of values already on the grid is exact, so the linear layer
equals the plain float64 product there.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """Value of each byte code (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def e4m3_encode(v) -> np.ndarray:
    """Byte code of float values: clamp to +-448, round to nearest even."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    out = np.zeros(a.shape, np.int64)
    sub = a < 2.0 ** -6
    # Subnormal range: multiples of 2^-9 (code = the multiple; 8 is 2^-6).
    out[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    n = ~sub
    if np.any(n):
        e = np.floor(np.log2(a[n])).astype(np.int64)
        q = np.rint(a[n] / 2.0 ** (e - 3)).astype(np.int64)  # 8 .. 16 (16 carries)
        carry = q == 16
        e = np.where(carry, e + 1, e)
        q = np.where(carry, 8, q)
        out[n] = ((e + 7) << 3) | (q - 8)
    out = np.where(v < 0, out | 0x80, out)
    return out.astype(np.uint8)


def quantize_rows(x):
    """Per-row E4M3 codes and float32 scales of a float32 matrix (see above)."""
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax)
    scale = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    prod = (x * inv[:, None]).astype(np.float32)
    return e4m3_encode(prod), scale


def linear_fp8(qa, sa, qw, sw, bias=None) -> np.ndarray:
    """y[r, n] = sum_k dec(qa[r, k]) dec(qw[n, k]) * sa[r] * sw[n] + bias[n]."""
    a = e4m3_decode(qa)
    w = e4m3_decode(qw)
    y = (a @ w.T) * np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y
