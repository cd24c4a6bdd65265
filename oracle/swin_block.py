"""CPU oracle for the full Swin block forward around the attention sub-layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with
the HIP library and imports nothing from it.

Plain float64 numpy.  The attention sub-layer is ``swin_oracle.wmsa_forward``;
this module adds what surrounds it in a transformer block:

  * "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization" --
    Section 3.2 / Figure 3: the Swin block is the standard transformer block
    with its multi-head attention replaced by shifted-window attention and the
    other layers kept (the feed-forward module's linear layers are GEMMs);
    Section 2.2 names GeLU among the activations of vision transformers.
  * "Boosting Swin Transformer Speed", Training Optimization: LayerNorm is part
    of the block (it is one of the fused operators).
  * "Swin Transformer V2" research summary, How It Works: V1 normalises before each sub-layer (pre-norm); V2 normalises
    each residual branch's output before it is added back (residual
    post-normalisation).

Readings (the pages are silent on these):
  * LayerNorm over the C channels of a token, biased variance, eps = 1e-5,
    per-channel gamma and beta.
  * MLP = Linear(C -> hidden) + bias, GELU, Linear(hidden -> C) + bias, with the
    exact (erf) GELU; hidden = 4C in the tests and the benchmark.
  * V1: h = x + A(LN1(x)),  y = h + F(LN2(h)).
    V2: h = x + LN1(A(x)),  y = h + LN2(F(h)).
    (A = the attention sub-layer, F = the MLP.)

Parity pins: closed forms and invariants in ``tests/test_oracle_block.py``
(LayerNorm moments, GELU values from the normal CDF, an identity block, uniform
attention over a single window, the two residual orders).
"""
from __future__ import annotations

import math

import numpy as np

from . import swin_oracle as so

LN_EPS = 1e-5


def layer_norm(x, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * gamma + beta,
    biased variance (the mean of squared deviations)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + \
        np.asarray(beta, np.float64)


_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu(x) -> np.ndarray:
    """Exact GELU: x * Phi(x), Phi the standard normal CDF = (1 + erf(x/sqrt 2)) / 2."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def mlp(x, w1, b1, w2, b2) -> np.ndarray:
    """Linear(C -> hidden) + bias, GELU, Linear(hidden -> C) + bias; weights in
    [out, in] layout, biases may be None (zeros)."""
    x = np.asarray(x, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    h = x @ w1.T
    if b1 is not None:
        h = h + np.asarray(b1, np.float64)
    o = gelu(h) @ w2.T
    if b2 is not None:
        o = o + np.asarray(b2, np.float64)
    return o


def block_forward(x, p: dict, M: int, s: int, heads: int, mode: str = "v1",
                  windows=None):
    """Full block forward.  x [B, H, W, C]; p holds the attention parameters
    (w_qkv, b_qkv, w_proj, b_proj, table, tau) and the block's own (ln1_g, ln1_b,
    ln2_g, ln2_b, fc1_w, fc1_b, fc2_w, fc2_b).

    With ``windows`` (global window indices as in ``wmsa_forward``) only the
    tokens of those windows are computed: returns (token_index, y_rows) -- the
    LayerNorms and the MLP act per token, so a token's output needs only its own
    window of the attention.
    """
    x = np.asarray(x, np.float64)
    B, H, W, C = x.shape

    def attn(u, win):
        return so.wmsa_forward(u, p["w_qkv"], p.get("b_qkv"), p["w_proj"], p.get("b_proj"),
                               p["table"], M, s, heads, mode, tau=p.get("tau"),
                               windows=win)

    def ffn(u):
        return mlp(u, p["fc1_w"], p.get("fc1_b"), p["fc2_w"], p.get("fc2_b"))

    if mode == "v1":
        ln1x = layer_norm(x, p["ln1_g"], p["ln1_b"])
        if windows is None:
            h = x + attn(ln1x, None)
            return h + ffn(layer_norm(h, p["ln2_g"], p["ln2_b"]))
        tok, a = attn(ln1x, windows)
        h = x.reshape(-1, C)[tok] + a
        return tok, h + ffn(layer_norm(h, p["ln2_g"], p["ln2_b"]))
    if mode == "v2":
        if windows is None:
            h = x + layer_norm(attn(x, None), p["ln1_g"], p["ln1_b"])
            return h + layer_norm(ffn(h), p["ln2_g"], p["ln2_b"])
        tok, a = attn(x, windows)
        h = x.reshape(-1, C)[tok] + layer_norm(a, p["ln1_g"], p["ln1_b"])
        return tok, h + layer_norm(ffn(h), p["ln2_g"], p["ln2_b"])
    raise ValueError("mode must be 'v1' or 'v2'")
