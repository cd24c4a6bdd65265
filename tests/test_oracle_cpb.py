"""Pins of the oracle's V2 continuous-position-bias table: closed forms, a constant
special case, range, and an independent torch module evaluation.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import swin_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_log_coords_closed_forms():
    with open(os.path.join(GOLDEN, "cpb_closed_forms.json")) as f:
        g = json.load(f)
    for M in (2, 7, 16, 24):
        c = so.cpb_log_coords(M)
        n = 2 * M - 1
        centre = (M - 1) * n + (M - 1)
        assert np.array_equal(c[centre], [g["g_zero"], g["g_zero"]])
        assert math.isclose(c[0, 0], -g["g_edge"], rel_tol=1e-15)       # delta = (-(M-1), -(M-1))
        assert math.isclose(c[n * n - 1, 1], g["g_edge"], rel_tol=1e-15)
        # dy-major order: row r holds dy = r // n - (M-1), dx = r % n - (M-1)
        assert np.all(np.sign(c[:, 0]) == np.sign(np.arange(n * n) // n - (M - 1)))
        assert np.all(np.sign(c[:, 1]) == np.sign(np.arange(n * n) % n - (M - 1)))
    c9 = so.cpb_log_coords(9)
    assert math.isclose(c9[(8 + 1) * 17 + 8, 0], g["g_unit_M9"], rel_tol=1e-15)
    # odd symmetry g(-u) = -g(u)
    c = so.cpb_log_coords(7)
    assert np.array_equal(c[::-1], -c)


def test_cpb_constant_when_first_layer_zero():
    rng = np.random.default_rng(2)
    heads, hid, M = 4, 512, 16
    b1 = rng.normal(0, 1, hid)
    w2 = rng.normal(0, 1 / math.sqrt(hid), (heads, hid))
    b2 = rng.normal(0, 1, heads)
    t = so.cpb_table(np.zeros((hid, 2)), b1, w2, b2, M)
    o = w2 @ np.maximum(b1, 0) + b2
    assert np.allclose(t, 16 / (1 + np.exp(-o))[None, :], rtol=1e-14)
    assert np.ptp(t, axis=0).max() == 0.0


@pytest.mark.parametrize("M", [7, 16, 24])
def test_cpb_range_and_torch_module(M):
    rng = np.random.default_rng(M)
    heads, hid = 16, 512
    w1 = rng.normal(0, 1, (hid, 2))
    b1 = rng.normal(0, 1, hid)
    w2 = rng.normal(0, 1 / math.sqrt(hid), (heads, hid))
    t = so.cpb_table(w1, b1, w2, None, M)
    assert t.shape == ((2 * M - 1) ** 2, heads)
    assert np.all((t > 0) & (t < 16))
    # independent evaluation: torch modules on coordinates built by torch
    lin1 = torch.nn.Linear(2, hid, dtype=torch.float64)
    lin2 = torch.nn.Linear(hid, heads, bias=False, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1)); lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2))
        r = torch.arange(-(M - 1), M, dtype=torch.float64)
        grid = torch.stack(torch.meshgrid(r, r, indexing="ij"), -1).reshape(-1, 2) * (8.0 / (M - 1))
        g = torch.sign(grid) * torch.log2(grid.abs() + 1.0) / 3.0
        ref = 16 * torch.sigmoid(lin2(torch.relu(lin1(g)))).numpy()
    assert np.max(np.abs(t - ref)) < 1e-12


def test_cpb_coord_scale_raw_reading():
    """coord_scale = 1 feeds raw offsets: edge maps to log2(M)/3."""
    M = 7
    c = so.cpb_log_coords(M, coord_scale=1.0)
    assert math.isclose(c[-1, 0], math.log2(M) / 3.0, rel_tol=1e-15)
