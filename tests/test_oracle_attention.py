"""Pins of the oracle's block forward against independent formulations: torch's
multi-head attention (global case), a dense-mask global attention built from the
no-wrap rule, a pure-Python per-token brute force, closed forms, invariants and
hand-worked fixtures.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import bruteforce, swin_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _params(rng, C, heads, M, mode, bias_std=0.1, w_std=0.3):
    p = dict(
        w_qkv=rng.normal(0, w_std, (3 * C, C)), b_qkv=rng.normal(0, bias_std, 3 * C),
        w_proj=rng.normal(0, w_std, (C, C)), b_proj=rng.normal(0, bias_std, C),
        table=rng.normal(0, 0.5, ((2 * M - 1) ** 2, heads)))
    p["tau"] = rng.uniform(0.005, 0.3, heads) if mode == "v2" else None
    return p


def _run(x, p, M, s, heads, mode, **kw):
    return so.wmsa_forward(x, p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                           M, s, heads, mode, tau=p["tau"], **kw)


# --- hand-worked fixtures ----------------------------------------------------

def test_handworked_bias_only():
    g = _golden("handworked_bias_only.json")
    M = g["M"]
    table = np.log(np.arange(1, (2 * M - 1) ** 2 + 1, dtype=np.float64))[:, None]
    y = so.wmsa_forward(np.array(g["x"], float), np.array(g["w_qkv"], float), None,
                        np.array(g["w_proj"], float), None, table, M, g["s"], g["heads"], "v1")
    assert np.allclose(y, np.array(g["y"]), rtol=0, atol=1e-14)


def test_handworked_window_equals_image_shifted():
    g = _golden("handworked_window_equals_image_shifted.json")
    M = g["M"]
    rng = np.random.default_rng(3)
    for mode in ("v1", "v2"):
        table = rng.normal(0, 1, ((2 * M - 1) ** 2, 1))
        y = so.wmsa_forward(np.array(g["x"], float), np.array(g["w_qkv"], float), None,
                            np.array(g["w_proj"], float), None, table, M, g["s"], 1, mode,
                            tau=np.array([0.05]))
        assert np.allclose(y, np.array(g["y"]), rtol=0, atol=1e-14)


# --- global attention: torch's multi-head attention ----------------------------

@pytest.mark.parametrize("H,heads,C", [(4, 1, 8), (6, 2, 8), (5, 4, 16)])
def test_global_case_is_torch_mha(H, heads, C):
    """s = 0, M = H = W and a zero table: the block is plain multi-head attention."""
    rng = np.random.default_rng(11 + H)
    p = _params(rng, C, heads, H, "v1")
    p["table"] = np.zeros_like(p["table"])
    x = rng.normal(0, 1, (2, H, H, C))
    y = _run(x, p, H, 0, heads, "v1")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    seq = t(x.reshape(2, H * H, C)).transpose(0, 1)  # [L, batch, E]
    ref, _ = torch.nn.functional.multi_head_attention_forward(
        seq, seq, seq, C, heads, t(p["w_qkv"]), t(p["b_qkv"]), None, None, False, 0.0,
        t(p["w_proj"]), t(p["b_proj"]), training=False, need_weights=False)
    ref = ref.transpose(0, 1).reshape(2, H, H, C).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


# --- dense-mask global formulation --------------------------------------------

def _dense_reference(x, p, M, s, heads, mode):
    """Whole-image attention with a dense [T, T] additive mask built from the no-wrap
    rule and the shifted-frame offsets; torch float64 matmuls."""
    B, H, W, C = x.shape
    d = C // heads
    T = H * W
    allowed = bruteforce.allowed_pairs(H, W, M, s)
    add = torch.full((T, T), float("-inf"), dtype=torch.float64)
    bias_h = torch.zeros((heads, T, T), dtype=torch.float64)
    table = torch.from_numpy(p["table"])
    for (y, xx), (y2, x2) in allowed:
        i, j = y * W + xx, y2 * W + x2
        dy = ((y - s) % H) - ((y2 - s) % H)
        dx = ((xx - s) % W) - ((x2 - s) % W)
        add[i, j] = 0.0
        bias_h[:, i, j] = table[(dy + M - 1) * (2 * M - 1) + (dx + M - 1)]
    xt = torch.from_numpy(x.reshape(B, T, C))
    qkv = xt @ torch.from_numpy(p["w_qkv"]).T + torch.from_numpy(p["b_qkv"])
    q, k, v = [qkv[..., i * C:(i + 1) * C].reshape(B, T, heads, d).transpose(1, 2) for i in range(3)]
    if mode == "v1":
        lg = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    else:
        qn = torch.nn.functional.normalize(q, dim=-1, eps=1e-12)
        kn = torch.nn.functional.normalize(k, dim=-1, eps=1e-12)
        tau = torch.clamp(torch.from_numpy(p["tau"]), min=0.01)
        lg = (qn @ kn.transpose(-1, -2)) / tau[None, :, None, None]
    lg = lg + bias_h[None] + add[None, None]
    o = torch.softmax(lg, dim=-1) @ v
    o = o.transpose(1, 2).reshape(B, T, C)
    y = o @ torch.from_numpy(p["w_proj"]).T + torch.from_numpy(p["b_proj"])
    return y.reshape(B, H, W, C).numpy()


@pytest.mark.parametrize("mode", ["v1", "v2"])
@pytest.mark.parametrize("B,H,W,M,s,heads,C", [
    (2, 8, 8, 4, 2, 2, 8), (1, 14, 14, 7, 3, 2, 8), (1, 12, 8, 4, 1, 1, 4),
    (1, 6, 6, 6, 3, 2, 8), (2, 9, 9, 3, 0, 1, 4)])
def test_oracle_equals_dense_mask_global(mode, B, H, W, M, s, heads, C):
    rng = np.random.default_rng(100 + H * 7 + s)
    p = _params(rng, C, heads, M, mode)
    x = rng.normal(0, 1, (B, H, W, C))
    y = _run(x, p, M, s, heads, mode)
    ref = _dense_reference(x, p, M, s, heads, mode)
    assert np.max(np.abs(y - ref)) < 1e-11


# --- pure-Python per-token brute force ----------------------------------------

@pytest.mark.parametrize("mode", ["v1", "v2"])
@pytest.mark.parametrize("H,W,M,s", [(6, 6, 3, 1), (8, 12, 4, 2), (12, 12, 6, 3), (7, 7, 7, 3)])
def test_oracle_equals_bruteforce(mode, H, W, M, s):
    rng = np.random.default_rng(H * 31 + W + s)
    heads, C = 2, 4
    p = _params(rng, C, heads, M, mode)
    x = rng.normal(0, 1, (1, H, W, C))
    y = _run(x, p, M, s, heads, mode)
    bf = np.array(bruteforce.wmsa_forward(x, p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"],
                                          p["table"], M, s, heads, mode, tau=p["tau"]))
    assert np.max(np.abs(y - bf)) < 1e-12


# --- invariants and closed forms ---------------------------------------------

@pytest.mark.parametrize("mode", ["v1", "v2"])
def test_softmax_rows_and_masked_zero(mode):
    rng = np.random.default_rng(5)
    B, H, W, M, s, heads, C = 2, 12, 12, 4, 2, 2, 8
    p = _params(rng, C, heads, M, mode)
    x = rng.normal(0, 1, (B, H, W, C))
    _, P, L = _run(x, p, M, s, heads, mode, return_attention=True)
    assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-12
    lab = np.tile(so.region_labels(H, W, M, s), (B, 1))
    allowed = lab[:, :, None] == lab[:, None, :]
    assert np.all(P[np.broadcast_to(~allowed[:, None], P.shape)] == 0.0)
    assert np.all(P[np.broadcast_to(allowed[:, None], P.shape)] > 0.0)


def test_cosine_logits_bounded_by_inverse_tau():
    rng = np.random.default_rng(9)
    B, H, W, M, s, heads, C = 1, 8, 8, 4, 2, 4, 16
    p = _params(rng, C, heads, M, "v2")
    p["tau"] = np.array([0.001, 0.01, 0.05, 1.0])  # first one is clipped up to 0.01
    x = rng.normal(0, 1, (B, H, W, C))
    _, _, L = _run(x, p, M, s, heads, "v2", return_attention=True)
    rel = so.relative_position_index(M)
    bias = p["table"][rel.reshape(-1)].reshape(M * M, M * M, heads).transpose(2, 0, 1)
    t_eff = np.maximum(p["tau"], 0.01)
    cos = (L - bias[None]) * t_eff[None, :, None, None]
    assert np.all(np.abs(cos) <= 1.0 + 1e-12)
    # q parallel to k (W_k = W_q, same bias) gives cos = 1 exactly on i = j
    p["w_qkv"][C:2 * C] = p["w_qkv"][:C]
    p["b_qkv"][C:2 * C] = p["b_qkv"][:C]
    _, _, L = _run(x, p, M, s, heads, "v2", return_attention=True)
    diag = np.einsum("whii->whi", L - bias[None])
    assert np.allclose(diag, (1.0 / t_eff)[None, :, None], rtol=1e-13, atol=0)


def _region_mean_closed_form(x, p, M, s, heads):
    """y_i = W_proj mean_{j allowed for i} v_j + b_proj, with allowed pairs from the
    no-wrap rule (uniform attention)."""
    B, H, W, C = x.shape
    v = x @ p["w_qkv"][2 * C:].T + p["b_qkv"][2 * C:]
    pairs = bruteforce.allowed_pairs(H, W, M, s)
    keys = {}
    for a, b in pairs:
        keys.setdefault(a, []).append(b)
    o = np.zeros_like(v)
    for (y, xx), ks in keys.items():
        o[:, y, xx] = np.mean([v[:, y2, x2] for (y2, x2) in ks], axis=0)
    return o @ p["w_proj"].T + p["b_proj"]


def test_uniform_attention_closed_forms():
    rng = np.random.default_rng(21)
    B, H, W, M, s, heads, C = 2, 8, 8, 4, 2, 2, 8
    x = rng.normal(0, 1, (B, H, W, C))
    # V1 with W_q = W_k = 0 and a zero table: uniform over each region
    p = _params(rng, C, heads, M, "v1")
    p["w_qkv"][:2 * C] = 0.0
    p["b_qkv"][:2 * C] = 0.0
    p["table"][:] = 0.0
    y = _run(x, p, M, s, heads, "v1")
    assert np.max(np.abs(y - _region_mean_closed_form(x, p, M, s, heads))) < 1e-12
    # V2 with a huge tau and a zero table: the cosine term vanishes
    p = _params(rng, C, heads, M, "v2")
    p["tau"] = np.full(heads, 1e12)
    p["table"][:] = 0.0
    y = _run(x, p, M, s, heads, "v2")
    assert np.max(np.abs(y - _region_mean_closed_form(x, p, M, s, heads))) < 1e-10


def test_bias_only_softmax_closed_form_and_one_hot():
    """W_q = 0: each row is softmax of its bias row over the allowed keys; a one-hot
    table entry at offset (dy, dx) = (1, 0) sends the weight to the key one row above
    the query (shifted frame)."""
    rng = np.random.default_rng(33)
    B, H, W, M, s, heads, C = 1, 8, 8, 4, 2, 1, 4
    x = rng.normal(0, 1, (B, H, W, C))
    p = _params(rng, C, heads, M, "v1")
    p["w_qkv"][:C] = 0.0
    p["b_qkv"][:C] = 0.0
    _, P, _ = _run(x, p, M, s, heads, "v1", return_attention=True)
    lab = so.region_labels(H, W, M, s)
    rel = so.relative_position_index(M)
    for w in range(lab.shape[0]):
        for i in range(M * M):
            js = [j for j in range(M * M) if lab[w, j] == lab[w, i]]
            e = np.array([math.exp(p["table"][rel[i, j], 0]) for j in js])
            assert np.allclose(P[w, 0, i, js], e / e.sum(), rtol=1e-13, atol=1e-15)
    p["table"][:] = 0.0
    p["table"][(1 + M - 1) * (2 * M - 1) + (M - 1), 0] = 60.0
    _, P, _ = _run(x, p, M, s, heads, "v1", return_attention=True)
    for w in range(lab.shape[0]):
        for i in range(M, M * M):
            j = i - M
            if lab[w, j] == lab[w, i]:
                assert P[w, 0, i, j] >= 1 - 1e-15
                assert np.all(np.delete(P[w, 0, i], j) < 1e-25)


def test_window_subset_matches_full():
    rng = np.random.default_rng(41)
    B, H, W, M, s, heads, C = 2, 12, 8, 4, 2, 2, 8
    for mode in ("v1", "v2"):
        p = _params(rng, C, heads, M, mode)
        x = rng.normal(0, 1, (B, H, W, C))
        y = _run(x, p, M, s, heads, mode)
        sel = [0, 3, 5, 11]
        tok, rows = _run(x, p, M, s, heads, mode, windows=sel)
        assert np.array_equal(rows, y.reshape(-1, C)[tok])
        assert len(set(tok.tolist())) == len(sel) * M * M


def test_scale_argument_and_tau_min():
    rng = np.random.default_rng(51)
    B, H, W, M, s, heads, C = 1, 4, 4, 2, 1, 2, 8
    p = _params(rng, C, heads, M, "v1")
    x = rng.normal(0, 1, (B, H, W, C))
    y_default = _run(x, p, M, s, heads, "v1")
    y_explicit = _run(x, p, M, s, heads, "v1", scale=(C // heads) ** -0.5)
    assert np.array_equal(y_default, y_explicit)
    p = _params(rng, C, heads, M, "v2")
    p["tau"] = np.array([0.001, 0.002])
    y1 = _run(x, p, M, s, heads, "v2")
    p["tau"] = np.array([0.01, 0.01])
    y2 = _run(x, p, M, s, heads, "v2")
    assert np.array_equal(y1, y2)
