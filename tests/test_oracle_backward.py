"""Pins of the backward oracle (oracle/swin_backward.py).

Central finite differences of L = sum(dy * y) through the forward oracle (itself
pinned by test_oracle_attention.py) on tiny inputs, for every input of the
sub-layer, V1 and V2, with and without the shift; closed forms: the projection
bias gradient is the sum of dy, and each head's table gradient sums to zero
(a softmax row does not change when one constant is added to all its logits,
and the table adds to every logit of a head).
"""
import numpy as np
import pytest

from oracle import swin_backward as sbw
from oracle import swin_oracle as so


def _case(seed, B, H, W, C, heads, M, mode, tau=None):
    r = np.random.default_rng(seed)
    p = {
        "x": r.normal(size=(B, H, W, C)),
        "w_qkv": r.normal(0, 0.4, (3 * C, C)),
        "b_qkv": r.normal(0, 0.2, 3 * C),
        "w_proj": r.normal(0, 0.4, (C, C)),
        "b_proj": r.normal(0, 0.2, C),
        "table": r.normal(0, 0.5, ((2 * M - 1) ** 2, heads)),
    }
    if mode == "v2":
        p["tau"] = np.asarray(tau, np.float64)
    dy = r.normal(size=(B, H, W, C))
    return p, dy


def _loss(p, dy, M, s, heads, mode):
    y = so.wmsa_forward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                        M, s, heads, mode, tau=p.get("tau"))
    return float((y * dy).sum())


def _fd_check(p, dy, M, s, heads, mode, name, gkey, n_samples, seed, h=1e-5, tol=2e-7):
    g = sbw.wmsa_backward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                          M, s, heads, dy, mode, tau=p.get("tau"))[gkey]
    arr = p[name]
    r = np.random.default_rng(seed)
    idx = [tuple(int(r.integers(0, n)) for n in arr.shape) for _ in range(n_samples)]
    scale = max(1.0, float(np.abs(g).max()))
    for i in idx:
        keep = arr[i]
        arr[i] = keep + h
        lp = _loss(p, dy, M, s, heads, mode)
        arr[i] = keep - h
        lm = _loss(p, dy, M, s, heads, mode)
        arr[i] = keep
        fd = (lp - lm) / (2 * h)
        assert abs(fd - g[i]) <= tol * scale, (name, i, fd, g[i])


GRADS = [("x", "dx"), ("w_qkv", "dw_qkv"), ("b_qkv", "db_qkv"), ("w_proj", "dw_proj"),
         ("b_proj", "db_proj"), ("table", "dtable")]


@pytest.mark.parametrize("s", [0, 2])
@pytest.mark.parametrize("name,gkey", GRADS)
def test_v1_finite_differences(name, gkey, s):
    p, dy = _case(11 + s, 1, 8, 8, 8, 2, 4, "v1")
    _fd_check(p, dy, 4, s, 2, "v1", name, gkey, n_samples=12, seed=5)


@pytest.mark.parametrize("s", [0, 2])
@pytest.mark.parametrize("name,gkey", GRADS + [("tau", "dtau")])
def test_v2_finite_differences(name, gkey, s):
    # tau of head 1 below the clamp: its gradient must be exactly zero.
    p, dy = _case(23 + s, 1, 8, 8, 8, 2, 4, "v2", tau=[0.5, 0.004])
    # 1/tau reaches 100 here: a smaller step keeps the difference's truncation
    # error (third derivative x h^2) below the bar.
    _fd_check(p, dy, 4, s, 2, "v2", name, gkey, n_samples=12, seed=6, h=1e-6)


def test_v2_clamped_tau_has_zero_gradient():
    p, dy = _case(3, 1, 8, 8, 8, 2, 4, "v2", tau=[0.3, 0.005])
    g = sbw.wmsa_backward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                          4, 2, 2, dy, "v2", tau=p["tau"])
    assert g["dtau"][1] == 0.0 and g["dtau"][0] != 0.0
    # the error scale of dtau: the same sum over |terms| bounds it, and is zero
    # where the clamp is flat
    assert g["dtau_abs"][1] == 0.0 and g["dtau_abs"][0] >= abs(g["dtau"][0]) > 0.0


@pytest.mark.parametrize("mode", ["v1", "v2"])
def test_closed_forms(mode):
    p, dy = _case(7, 2, 12, 8, 12, 3, 4, mode, tau=[0.2, 0.05, 1.0])
    g = sbw.wmsa_backward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                          4, 2, 3, dy, mode, tau=p.get("tau"))
    np.testing.assert_allclose(g["db_proj"], dy.sum(axis=(0, 1, 2)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dtable"].sum(axis=0), 0.0, atol=1e-10)
    # Shapes of every gradient match their inputs.
    for name, gkey in GRADS:
        assert g[gkey].shape == np.shape(p[name]), gkey


def test_window_equal_to_image_is_plain_attention_backward():
    # One window covering the image, no shift: the sub-layer is global MHA with a
    # bias, whose gradient a hand-written loop over tokens reproduces.
    p, dy = _case(9, 1, 3, 3, 4, 1, 3, "v1")
    g = sbw.wmsa_backward(p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"],
                          3, 0, 1, dy, "v1")
    x = p["x"].reshape(9, 4)
    q = x @ p["w_qkv"][:4].T + p["b_qkv"][:4]
    k = x @ p["w_qkv"][4:8].T + p["b_qkv"][4:8]
    v = x @ p["w_qkv"][8:].T + p["b_qkv"][8:]
    rel = so.relative_position_index(3)
    dv = np.zeros_like(v)
    dS = np.zeros((9, 9))
    do = dy.reshape(9, 4) @ p["w_proj"]
    for i in range(9):
        lg = np.array([q[i] @ k[j] / 2.0 + p["table"][rel[i, j], 0] for j in range(9)])
        pr = np.exp(lg - lg.max())
        pr /= pr.sum()
        dp = np.array([do[i] @ v[j] for j in range(9)])
        for j in range(9):
            dv[j] += pr[j] * do[i]
            dS[i, j] = pr[j] * (dp[j] - (pr * dp).sum())
    dq = dS @ k / 2.0
    dk = dS.T @ q / 2.0
    dqkv = np.concatenate([dq, dk, dv], axis=1)
    np.testing.assert_allclose(g["dx"].reshape(9, 4), dqkv @ p["w_qkv"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dw_qkv"], dqkv.T @ x, rtol=1e-10, atol=1e-12)
    dtab = np.zeros(25)
    for i in range(9):
        for j in range(9):
            dtab[rel[i, j]] += dS[i, j]
    np.testing.assert_allclose(g["dtable"][:, 0], dtab, rtol=1e-10, atol=1e-12)


def test_cpb_backward_finite_differences():
    r = np.random.default_rng(4)
    M, hid, heads = 4, 16, 3
    w1, b1 = r.normal(size=(hid, 2)), r.normal(size=hid)
    w2, b2 = r.normal(0, 0.3, (heads, hid)), r.normal(size=heads)
    dt = r.normal(size=((2 * M - 1) ** 2, heads))
    g = sbw.cpb_backward(w1, b1, w2, b2, M, dt)

    def L():
        return float((so.cpb_table(w1, b1, w2, b2, M) * dt).sum())

    for arr, key in ((w1, "dw1"), (b1, "db1"), (w2, "dw2"), (b2, "db2")):
        for i in [tuple(int(r.integers(0, n)) for n in arr.shape) for _ in range(6)]:
            keep = arr[i]
            arr[i] = keep + 1e-6
            lp = L()
            arr[i] = keep - 1e-6
            lm = L()
            arr[i] = keep
            assert abs((lp - lm) / 2e-6 - g[key][i]) <= 1e-6 * max(1.0, abs(g[key][i])), (key, i)


@pytest.mark.parametrize("mode,s", [("v1", 2), ("v2", 2), ("v1", 0)])
def test_window_subset_matches_whole_image(mode, s):
    # A window subset gives the whole image's dx at its windows' tokens, and
    # the partial sums of two complementary subsets add up to the whole
    # image's gradients (windows are independent given the weights).
    M, heads = 4, 2
    p, dy = _case(12, 2, 8, 12, 16, heads, M, mode, tau=[0.3, 0.02])
    args = (p["x"], p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"], M, s, heads,
            dy, mode)
    full = sbw.wmsa_backward(*args, tau=p.get("tau"))
    nwin = 2 * (8 // M) * (12 // M)
    a = [0, 3, 5, nwin - 1]                # includes masked (last row / column) windows
    b = [w for w in range(nwin) if w not in a]
    ga = sbw.wmsa_backward(*args, tau=p.get("tau"), windows=a)
    gb = sbw.wmsa_backward(*args, tau=p.get("tau"), windows=b)
    src = so.window_token_source(2, 8, 12, M, s)          # [windows, N] flat token
    dx_flat = full["dx"].reshape(-1, 16)
    np.testing.assert_allclose(ga["dxw"], dx_flat[src[a]], rtol=1e-12, atol=1e-12)
    for k in ("dw_qkv", "db_qkv", "dw_proj", "db_proj", "dtable") + (("dtau",) if mode == "v2"
                                                                     else ()):
        np.testing.assert_allclose(ga[k] + gb[k], full[k], rtol=1e-10, atol=1e-10)
    assert "dx" not in ga
