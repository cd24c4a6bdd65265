"""Support of the 16-bit parity bar of the full block (helpers.assert_block_close),
on the CPU: an implementation that is exact except for rounding what it stores
in the I/O type -- the attention output (carrying the attention sub-layer's own
allowed error), each LayerNorm output, the MLP hidden layer, the residual
stream h and y -- stays inside the bar with margin, and a dropped term does not.

The emulation follows the unfused sequence of swin_block_fwd (the most stored
roundings; the fused MLP keeps h and the LayerNorm output in float32):
  V1: a = LN1(x); b = A(a); h = x + b; c = LN2(h); u = GELU(c W1^T + b1);
      y = u W2^T + b2 + h
  V2: b = A(x); h = x + LN1(b); u = GELU(h W1^T + b1); f = u W2^T + b2;
      y = h + LN2(f)
every named intermediate rounded float64 -> float32 -> the I/O type (round to
nearest even), as the kernels store it."""
import numpy as np
import pytest
import torch

import workloads
from oracle import swin_block as sb
from oracle import swin_oracle as so

import helpers


def _round(a, dtype):
    t = torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32)
    return t.to(workloads.DTYPES[dtype]).to(torch.float64).numpy()


def _emulated_block(x, p, M, s, heads, mode, dtype, rng, drop=None):
    """The block with its stored roundings.  The attention output also gets
    Gaussian noise for the attention sub-layer's own error: its three stored
    roundings (q / k / v, P, O), each uniform within a half-ulp u (RMS
    u / sqrt 3), add up in quadrature to a relative RMS of about u; capped by
    the sub-layer's parity bars (relative L2 5e-3; max-abs 2e-2 at 5 sigma).
    ``drop`` plants a mistake: "ln2_b" leaves out LayerNorm 2's shift, "gelu"
    uses ReLU for GELU, "resid" adds x instead of h as the second residual."""
    R = lambda a: _round(a, dtype)

    def attn(u):
        a = so.wmsa_forward(u, p["w_qkv"], p["b_qkv"], p["w_proj"], p["b_proj"], p["table"], M, s,
                            heads, mode, tau=p.get("tau"))
        u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
        sigma = min(min(u, 5e-3) * np.sqrt(np.mean(a ** 2)), 2e-2 / 5)
        noise = rng.standard_normal(a.shape) * sigma
        return R(a + noise)

    ln2_b = np.zeros_like(p["ln2_b"]) if drop == "ln2_b" else p["ln2_b"]
    act = (lambda v: np.maximum(v, 0.0)) if drop == "gelu" else sb.gelu

    def ffn_hidden(u):
        return R(act(u @ p["fc1_w"].T + p["fc1_b"]))

    if mode == "v1":
        a = R(sb.layer_norm(x, p["ln1_g"], p["ln1_b"]))
        h = R(x + attn(a))
        c = R(sb.layer_norm(h, p["ln2_g"], ln2_b))
        return R(ffn_hidden(c) @ p["fc2_w"].T + p["fc2_b"] + (x if drop == "resid" else h))
    h = R(x + R(sb.layer_norm(attn(x), p["ln1_g"], p["ln1_b"])))
    f = R(ffn_hidden(h) @ p["fc2_w"].T + p["fc2_b"])
    return R((x if drop == "resid" else h) + sb.layer_norm(f, p["ln2_g"], ln2_b))


def _case(C, dtype, mode, seed):
    # The recipe of the GPU block parity cases (tests/test_gpu_block.py).
    heads, M, s = C // 32, 8, 4
    case = workloads.make_case(1, 16, 16, C, heads, M, (s,), dtype, mode, seed=seed, w_std=0.08,
                               bias_std=0.05, tau="uniform")
    blk = case.blocks[0]
    extra = workloads.make_block_params(C, dtype, seed + 1, fc_std=0.02)
    p = {"w_qkv": workloads.f64(blk.w_qkv), "b_qkv": workloads.f64(blk.b_qkv),
         "w_proj": workloads.f64(blk.w_proj), "b_proj": workloads.f64(blk.b_proj),
         "table": helpers.oracle_table(case, blk)}
    if mode == "v2":
        p["tau"] = workloads.f64(blk.tau)
    p.update({k: workloads.f64(v) for k, v in extra.items()})
    return workloads.f64(case.x), p, M, s, heads


@pytest.mark.parametrize("C", [96, 512])
@pytest.mark.parametrize("mode", ["v1", "v2"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rounding_emulation_inside_bar(C, mode, dtype):
    x, p, M, s, heads = _case(C, dtype, mode, seed=C + len(mode))
    ref = sb.block_forward(x, p, M, s, heads, mode)
    y = _emulated_block(x, p, M, s, heads, mode, dtype, np.random.default_rng(1))
    worst, rel = helpers.assert_block_close(y, ref, dtype, "emulated")
    # margin: the emulated errors use at most 90 % of the per-element bar and
    # 60 % of the rel-L2 bar
    assert worst <= 0.9, worst
    assert rel <= 0.6e-2, rel


# (V1 with these weights: LayerNorm 2's shift moves the MLP branch by less than
# the bar, so it is not a mistake the bar can see there.)
@pytest.mark.parametrize("mode,drop", [("v1", "gelu"), ("v1", "resid"), ("v2", "gelu"),
                                       ("v2", "resid"), ("v2", "ln2_b")])
def test_planted_mistake_breaks_bar(mode, drop):
    x, p, M, s, heads = _case(128, "bf16", mode, seed=7)
    ref = sb.block_forward(x, p, M, s, heads, mode)
    y = _emulated_block(x, p, M, s, heads, mode, "bf16", np.random.default_rng(2), drop=drop)
    with pytest.raises(AssertionError):
        helpers.assert_block_close(y, ref, "bf16", "planted")
