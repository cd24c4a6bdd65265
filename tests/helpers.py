"""Shared test helpers: run a seeded case through the HIP path (via the C ABI
binding) and through the CPU oracle, and compare them."""
from __future__ import annotations

import numpy as np
import torch

import workloads
from oracle import swin_oracle as so

# Parity bars: float32 I/O max-abs <= 1e-4; 16-bit I/O (float32 accumulation)
# max-abs <= 2e-2 and relative L2 <= 5e-3.
TOL_F32_MAXABS = 1e-4
TOL_16_MAXABS = 2e-2
TOL_16_RELL2 = 5e-3


def gpu_table(case: workloads.Case, blk: workloads.BlockParams, dev="cuda") -> torch.Tensor:
    import shifted_window_attention_roll_amd as swin
    if case.mode == "v1":
        return blk.table.to(dev)
    return swin.cpb_table(blk.cpb_w1.to(dev), blk.cpb_b1.to(dev), blk.cpb_w2.to(dev),
                          blk.cpb_b2.to(dev), case.M)


def oracle_table(case: workloads.Case, blk: workloads.BlockParams) -> np.ndarray:
    if case.mode == "v1":
        return workloads.f64(blk.table)
    return so.cpb_table(workloads.f64(blk.cpb_w1), workloads.f64(blk.cpb_b1),
                        workloads.f64(blk.cpb_w2), workloads.f64(blk.cpb_b2), case.M)


def run_gpu_block(case, blk, x_dev: torch.Tensor, out=None, workspace=None) -> torch.Tensor:
    import shifted_window_attention_roll_amd as swin
    dev = x_dev.device
    return swin.wmsa_fwd(x_dev, blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev),
                         blk.b_proj.to(dev), gpu_table(case, blk, dev), case.M, blk.s, case.heads,
                         case.mode, tau=None if blk.tau is None else blk.tau.to(dev), out=out,
                         workspace=workspace)


def run_oracle_block(case, blk, x64: np.ndarray, windows=None):
    return so.wmsa_forward(x64, workloads.f64(blk.w_qkv), workloads.f64(blk.b_qkv),
                           workloads.f64(blk.w_proj), workloads.f64(blk.b_proj),
                           oracle_table(case, blk), case.M, blk.s, case.heads, case.mode,
                           tau=None if blk.tau is None else workloads.f64(blk.tau),
                           windows=windows)


def errors(y: np.ndarray, ref: np.ndarray):
    d = y - ref
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
    return maxabs, rel


def assert_close(y: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    maxabs, rel = errors(y, ref)
    if dtype == "fp32":
        assert maxabs <= TOL_F32_MAXABS, f"{what}: max-abs {maxabs:.3e} > {TOL_F32_MAXABS}"
    else:
        assert maxabs <= TOL_16_MAXABS, f"{what}: max-abs {maxabs:.3e} > {TOL_16_MAXABS}"
        assert rel <= TOL_16_RELL2, f"{what}: rel-L2 {rel:.3e} > {TOL_16_RELL2}"
    return maxabs, rel


def sample_windows(B: int, H: int, W: int, M: int, n_random: int, seed: int):
    """Window ids: first, last, the last row / column of the first and last image
    (masked when shifted) and a seeded random handful."""
    nWy, nWx = H // M, W // M
    nW = nWy * nWx
    picks = {0, B * nW - 1, nWx - 1, nW - nWx, nW - 1, (B - 1) * nW}
    rng = np.random.default_rng(seed)
    picks.update(int(v) for v in rng.integers(0, B * nW, n_random))
    return sorted(p for p in picks if 0 <= p < B * nW)


def assert_block_close(y, ref, dtype, what):
    """float32: the attention's bar (max-abs 1e-4).  16-bit: the block stores
    its intermediates in the I/O type, so on top of the attention's bar (2e-2
    absolute) each element carries (a) the rounding of h and of y, two
    half-ulps of its own magnitude (half-ulp u = 2^-8 relative for bfloat16,
    2^-11 for float16), and (b) roundings made before a LayerNorm or inside the
    MLP (the attention output, a LayerNorm output, the hidden layer), which
    scale with the token's RMS, about five such units; so per element
    |err| <= 2e-2 + 2u |ref| + 5u RMS(ref row).  Overall rel-L2 <= 1e-2: the
    attention sub-layer's own 5e-3 plus five stored roundings of about
    u / (2 sqrt 3) RMS each (bfloat16: 1.1e-3; in quadrature 2.5e-3), with
    margin."""
    if dtype == "fp32":
        assert_close(y, ref, dtype, what)
        return
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    C = ref.shape[-1]
    yr, rr = y.reshape(-1, C), ref.reshape(-1, C)
    err = np.abs(yr - rr)
    bound = 2e-2 + 2 * u * np.abs(rr) + 5 * u * np.sqrt((rr ** 2).mean(axis=1, keepdims=True))
    i = int(np.argmax(err / bound))
    assert np.all(err <= bound), f"{what}: |err| {err.flat[i]:.3e} > {bound.flat[i]:.3e}"
    maxabs, rel = errors(y, ref)
    assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e}"
    return float(np.max(err / bound)), rel
