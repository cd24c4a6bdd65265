"""Pins of the block oracle (oracle/swin_block.py) against closed forms and
invariants: LayerNorm moments, GELU values of the normal CDF, the MLP as two
textbook matmuls, an identity block, uniform attention over one window, and the
two residual orders (V1 pre-norm, V2 post-norm)."""
import math

import numpy as np
import pytest

from oracle import swin_block as sb

RNG = np.random.default_rng(1234)


def test_layer_norm_moments():
    x = RNG.normal(3.0, 5.0, (7, 96))
    y = sb.layer_norm(x, np.ones(96), np.zeros(96))
    np.testing.assert_allclose(y.mean(axis=-1), 0.0, atol=1e-12)
    # variance 1 up to the eps: var(y) = var / (var + eps)
    var = x.var(axis=-1)
    np.testing.assert_allclose(y.var(axis=-1), var / (var + sb.LN_EPS), rtol=1e-12)
    g, b = RNG.normal(size=96), RNG.normal(size=96)
    np.testing.assert_allclose(sb.layer_norm(x, g, b), y * g + b, rtol=1e-12, atol=1e-12)


def test_layer_norm_constant_row_gives_beta():
    b = RNG.normal(size=32)
    np.testing.assert_allclose(sb.layer_norm(np.full((3, 32), 2.5), np.ones(32), b),
                               np.broadcast_to(b, (3, 32)), atol=1e-12)


def test_gelu_values():
    # x * Phi(x) with Phi(1) = 0.8413447460685429 (standard normal CDF table value).
    phi1 = 0.8413447460685429
    np.testing.assert_allclose(sb.gelu(np.array([0.0, 1.0, -1.0])),
                               [0.0, phi1, -(1.0 - phi1)], rtol=0, atol=1e-15)
    x = RNG.normal(0, 3, 1000)
    np.testing.assert_allclose(sb.gelu(x) - sb.gelu(-x), x, atol=1e-12)  # Phi(x)+Phi(-x) = 1
    np.testing.assert_allclose(sb.gelu(np.array([12.0, -12.0])), [12.0, 0.0], atol=1e-12)


def test_mlp_is_two_matmuls():
    x = RNG.normal(size=(5, 32))
    w1, b1 = RNG.normal(size=(128, 32)), RNG.normal(size=128)
    w2, b2 = RNG.normal(size=(32, 128)), RNG.normal(size=32)
    h = np.array([[sum(x[t, k] * w1[n, k] for k in range(32)) + b1[n] for n in range(128)]
                  for t in range(5)])
    g = np.array([[v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in row] for row in h])
    o = np.array([[sum(g[t, k] * w2[n, k] for k in range(128)) + b2[n] for n in range(32)]
                  for t in range(5)])
    np.testing.assert_allclose(sb.mlp(x, w1, b1, w2, b2), o, rtol=1e-10, atol=1e-10)


def _params(C, heads, M, mode, zero_attn=False, zero_mlp=False):
    R = 2 * M - 1
    p = dict(w_qkv=RNG.normal(0, 0.2, (3 * C, C)), b_qkv=RNG.normal(0, 0.1, 3 * C),
             w_proj=RNG.normal(0, 0.2, (C, C)), b_proj=RNG.normal(0, 0.1, C),
             table=RNG.normal(0, 0.3, (R * R, heads)),
             ln1_g=RNG.normal(1, 0.2, C), ln1_b=RNG.normal(0, 0.2, C),
             ln2_g=RNG.normal(1, 0.2, C), ln2_b=RNG.normal(0, 0.2, C),
             fc1_w=RNG.normal(0, 0.2, (4 * C, C)), fc1_b=RNG.normal(0, 0.1, 4 * C),
             fc2_w=RNG.normal(0, 0.2, (C, 4 * C)), fc2_b=RNG.normal(0, 0.1, C))
    if mode == "v2":
        p["tau"] = RNG.uniform(0.05, 0.5, heads)
    if zero_attn:
        p["w_proj"] = np.zeros((C, C))
        p["b_proj"] = np.zeros(C)
    if zero_mlp:
        p["fc2_w"] = np.zeros((C, 4 * C))
        p["fc2_b"] = np.zeros(C)
    return p


def test_identity_block_v1():
    # Pre-norm with both residual branches zero: y = x exactly.
    x = RNG.normal(size=(2, 8, 8, 64))
    p = _params(64, 2, 4, "v1", zero_attn=True, zero_mlp=True)
    np.testing.assert_allclose(sb.block_forward(x, p, 4, 2, 2, "v1"), x, atol=1e-12)


def test_zero_branches_v2():
    # Post-norm: a zero branch output is normalised to beta, so y = x + b1 + b2.
    x = RNG.normal(size=(1, 8, 8, 64))
    p = _params(64, 2, 4, "v2", zero_attn=True, zero_mlp=True)
    np.testing.assert_allclose(sb.block_forward(x, p, 4, 0, 2, "v2"),
                               x + p["ln1_b"] + p["ln2_b"], atol=1e-12)


def _uniform_attention_block(x, p, mode):
    """One window covering the image, no shift, zero q weights and table: every
    query averages every key, so the attention output of each token is
    W_proj (W_v mean(u) + b_v) + b_proj (u = the attention's input)."""
    C = x.shape[-1]
    wv, bv = p["w_qkv"][2 * C:], p["b_qkv"][2 * C:]

    def attn(u):
        m = u.reshape(-1, C).mean(axis=0)
        return np.broadcast_to(p["w_proj"] @ (wv @ m + bv) + p["b_proj"], u.shape)

    def ln(u, g, b):
        mu = u.mean(-1, keepdims=True)
        return (u - mu) / np.sqrt(((u - mu) ** 2).mean(-1, keepdims=True) + 1e-5) * g + b

    def ffn(u):
        h = u @ p["fc1_w"].T + p["fc1_b"]
        g = h * 0.5 * (1 + np.vectorize(math.erf)(h / math.sqrt(2)))
        return g @ p["fc2_w"].T + p["fc2_b"]

    if mode == "v1":
        h = x + attn(ln(x, p["ln1_g"], p["ln1_b"]))
        return h + ffn(ln(h, p["ln2_g"], p["ln2_b"]))
    h = x + ln(attn(x), p["ln1_g"], p["ln1_b"])
    return h + ln(ffn(h), p["ln2_g"], p["ln2_b"])


@pytest.mark.parametrize("mode", ["v1", "v2"])
def test_uniform_attention_block(mode):
    C, heads, M = 64, 2, 6
    x = RNG.normal(size=(1, M, M, C))
    p = _params(C, heads, M, mode)
    p["w_qkv"][:C] = 0.0     # q = b_q: V1 logits q.k are then key-dependent ...
    p["b_qkv"][:C] = 0.0     # ... unless q = 0 as well
    p["table"][:] = 0.0
    if mode == "v2":
        p["w_qkv"][C:2 * C] = 0.0  # cosine of q = 0 with anything is 0 (eps clamp)
        p["b_qkv"][C:2 * C] = 1.0
    np.testing.assert_allclose(sb.block_forward(x, p, M, 0, heads, mode),
                               _uniform_attention_block(x, p, mode), rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("mode", ["v1", "v2"])
def test_window_sampling_matches_full(mode):
    x = RNG.normal(size=(2, 8, 8, 32))
    p = _params(32, 1, 4, mode)
    full = sb.block_forward(x, p, 4, 2, 1, mode)
    tok, rows = sb.block_forward(x, p, 4, 2, 1, mode, windows=[1, 6])
    np.testing.assert_allclose(rows, full.reshape(-1, 32)[tok], rtol=1e-12, atol=1e-12)


def test_residual_orders_differ():
    # The same parameters give different blocks under the two norm placements
    # (a swapped placement would fail the uniform-attention pins above too).
    x = RNG.normal(size=(1, 8, 8, 32))
    p1 = _params(32, 1, 4, "v1")
    p2 = dict(p1, tau=np.full(1, 0.3))
    assert not np.allclose(sb.block_forward(x, p1, 4, 0, 1, "v1"),
                           sb.block_forward(x, p2, 4, 0, 1, "v2"))
