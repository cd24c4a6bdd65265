"""GPU parity of the full block forward (swin_block_fwd: LayerNorms, attention,
MLP, residuals) against the float64 oracle of oracle/swin_block.py."""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workloads
from oracle import swin_block as sb

import helpers

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import shifted_window_attention_roll_amd as swin
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    swin.load_library()
    return swin


def _say(msg):
    print(msg, flush=True)


def _assert_block_close(y, ref, dtype, what):
    helpers.assert_block_close(y, ref, dtype, what)


def _setup(B, H, W, C, heads, M, s, dtype, mode, seed, hidden=None):
    # MLP weights: N(0, 0.02) in 16 bits (the recipe of the attention weights;
    # the MLP branch is then 5-10 % of the residual stream), N(0, 0.1) in float32
    # (an O(1) branch, checked at the float32 bar).
    case = workloads.make_case(B, H, W, C, heads, M, (s,), dtype, mode, seed=seed, w_std=0.08,
                               bias_std=0.05, tau="uniform")
    blk = case.blocks[0]
    extra = workloads.make_block_params(C, dtype, seed + 1, hidden=hidden,
                                        fc_std=0.1 if dtype == "fp32" else 0.02)
    dev = "cuda"
    gp = {"w_qkv": blk.w_qkv.to(dev), "b_qkv": blk.b_qkv.to(dev), "w_proj": blk.w_proj.to(dev),
          "b_proj": blk.b_proj.to(dev), "table": helpers.gpu_table(case, blk, dev)}
    if mode == "v2":
        gp["tau"] = blk.tau.to(dev)
    gp.update({k: v.to(dev) for k, v in extra.items()})
    op = {"w_qkv": workloads.f64(blk.w_qkv), "b_qkv": workloads.f64(blk.b_qkv),
          "w_proj": workloads.f64(blk.w_proj), "b_proj": workloads.f64(blk.b_proj),
          "table": helpers.oracle_table(case, blk)}
    if mode == "v2":
        op["tau"] = workloads.f64(blk.tau)
    op.update({k: workloads.f64(v) for k, v in extra.items()})
    return case, blk, gp, op


@pytest.mark.parametrize("B,H,W,C,heads,M,s,dtype,mode", [
    (2, 14, 14, 96, 3, 7, 3, "fp16", "v1"),     # fused window-7 attention; fc2 N = 96
    (1, 14, 14, 96, 3, 7, 3, "fp32", "v1"),     # float32 throughout
    (1, 10, 10, 64, 2, 5, 2, "fp32", "v2"),     # 100 tokens: a ragged 128-row tile
    (2, 16, 16, 128, 4, 8, 4, "bf16", "v2"),    # fused window-8 attention
    (1, 32, 32, 128, 4, 16, 8, "bf16", "v2"),   # fused window-16 attention
    (1, 14, 14, 512, 16, 7, 3, "bf16", "v1"),   # C = 512: 8 channels per lane in LayerNorm
    (1, 14, 14, 512, 16, 7, 3, "fp32", "v1"),   # hidden 2048: long K in float32
    (1, 16, 24, 256, 8, 8, 3, "fp16", "v2"),    # tiled attention between the GEMMs
    (1, 10, 10, 64, 2, 5, 2, "bf16", "v1"),     # fused MLP, C = 64, 100 rows (ragged)
    (3, 7, 7, 32, 1, 7, 3, "fp16", "v2"),       # fused MLP, C = 32, 147 rows
])
def test_block_small(gpu, B, H, W, C, heads, M, s, dtype, mode):
    _say(f"block B={B} H={H} W={W} C={C} heads={heads} M={M} s={s} {dtype} {mode}")
    case, blk, gp, op = _setup(B, H, W, C, heads, M, s, dtype, mode, seed=C + 7 * M + s)
    y = gpu.block_fwd(case.x.cuda(), gp, M, s, heads, mode)
    torch.cuda.synchronize()
    ref = sb.block_forward(workloads.f64(case.x), op, M, s, heads, mode)
    _assert_block_close(workloads.f64(y.cpu()), ref, dtype, "block")


def test_block_swin_t_stage1_sampled(gpu):
    # Swin-T stage 1 at B = 64 (fp16, V1, shift 3): sampled windows, every corner.
    B, H, W, C, heads, M, s = 64, 56, 56, 96, 3, 7, 3
    _say("block Swin-T stage 1 B=64 fp16 v1 sampled")
    case, blk, gp, op = _setup(B, H, W, C, heads, M, s, "fp16", "v1", seed=2024)
    y = gpu.block_fwd(case.x.cuda(), gp, M, s, heads, "v1")
    torch.cuda.synchronize()
    wins = helpers.sample_windows(B, H, W, M, 24, seed=5)
    tok, ref = sb.block_forward(workloads.f64(case.x), op, M, s, heads, "v1", windows=wins)
    got = workloads.f64(y.cpu()).reshape(-1, C)[tok]
    _assert_block_close(got, ref, "fp16", "block sampled")


@pytest.mark.parametrize("name,n_random", [
    ("swin_b_stage3_b64_bf16", 12),          # C = 512: MLP on the tiled dense GEMMs
    ("swinv2_b_stage1_w16_bf16", 12),        # C = 128: the fused MLP, window-16 block kernel
    ("swinv2_g_stage1_384_w24_bf16", 6),     # C = 512, window 24, hidden 2048
])
def test_block_workload_sampled(gpu, name, n_random):
    # The full block on the workload's last block with the MLP weights the
    # bench times it with: sampled windows (first, last, the masked last row /
    # column and a seeded handful) against the oracle run on those windows.
    _say(f"block {name} sampled")
    case = workloads.make_workload(name)
    blk = case.blocks[-1]
    M, s, heads, C = case.M, blk.s, case.heads, case.C
    extra = workloads.make_block_params(C, case.dtype, 77, fc_std=0.02)
    dev = "cuda"
    gp = {"w_qkv": blk.w_qkv.to(dev), "b_qkv": blk.b_qkv.to(dev), "w_proj": blk.w_proj.to(dev),
          "b_proj": blk.b_proj.to(dev), "table": helpers.gpu_table(case, blk, dev)}
    op = {"w_qkv": workloads.f64(blk.w_qkv), "b_qkv": workloads.f64(blk.b_qkv),
          "w_proj": workloads.f64(blk.w_proj), "b_proj": workloads.f64(blk.b_proj),
          "table": helpers.oracle_table(case, blk)}
    if blk.tau is not None:
        gp["tau"] = blk.tau.to(dev)
        op["tau"] = workloads.f64(blk.tau)
    gp.update({k: v.to(dev) for k, v in extra.items()})
    op.update({k: workloads.f64(v) for k, v in extra.items()})
    x = case.x.to(dev)
    out = torch.full_like(x, float("nan"))
    y = gpu.block_fwd(x, gp, M, s, heads, case.mode, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    wins = helpers.sample_windows(case.B, case.H, case.W, M, n_random, seed=11)
    tok, ref = sb.block_forward(workloads.f64(case.x), op, M, s, heads, case.mode, windows=wins)
    got = workloads.f64(y.cpu()).reshape(-1, C)[tok]
    _assert_block_close(got, ref, case.dtype, f"block {name} sampled")


def test_block_deterministic_and_written(gpu):
    case, blk, gp, op = _setup(2, 16, 16, 128, 4, 8, 4, "bf16", "v2", seed=99)
    x = case.x.cuda()
    out = torch.full_like(x, float("nan"))
    y1 = gpu.block_fwd(x, gp, 8, 4, 4, "v2", out=out).clone()
    out.fill_(float("nan"))
    y2 = gpu.block_fwd(x, gp, 8, 4, 4, "v2", out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(y1.float()).all()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("C,heads,dtype,mode,hidden", [
    (64, 2, "bf16", "v1", 32),     # one hidden chunk
    (64, 2, "fp16", "v2", 160),    # hidden not 4C
    (128, 4, "bf16", "v1", 96),    # LDS-staged weights, three chunks
    (96, 3, "fp16", "v1", 544),    # 17 chunks
])
def test_block_fused_mlp_hidden_widths(gpu, C, heads, dtype, mode, hidden):
    _say(f"block fused MLP C={C} hidden={hidden} {dtype} {mode}")
    M = 8 if C != 96 else 7
    H = W = 2 * M
    case, blk, gp, op = _setup(2, H, W, C, heads, M, M // 2, dtype, mode, seed=C + hidden,
                               hidden=hidden)
    y = gpu.block_fwd(case.x.cuda(), gp, M, M // 2, heads, mode)
    torch.cuda.synchronize()
    ref = sb.block_forward(workloads.f64(case.x), op, M, M // 2, heads, mode)
    _assert_block_close(workloads.f64(y.cpu()), ref, dtype, "block hidden")
