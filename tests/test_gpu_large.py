"""GPU parity above 2 GiB of activations: the tiled GEMMs (32-bit buffer
offsets) hand over to the general kernels there.  One seeded 96 x 96 x 512
image (window 24, shift 12, V2, bfloat16) is repeated over a batch of 232
(2.19 GB of x): every image's output must equal image 0's bit for bit, and
image 0 must match the oracle -- for the attention sub-layer and for the full
block (its MLP layers then also run on the general dense kernel)."""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import swin_block as sb

import helpers

pytestmark = pytest.mark.gpu

B, H, W, C, HEADS, M, S = 232, 96, 96, 512, 16, 24, 12


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shifted_window_attention_roll_amd as swin
    swin.load_library()
    return swin


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _same_as_first(y):
    first = y[0:1].view(torch.int16)
    for b0 in range(0, y.shape[0], 32):
        chunk = y[b0:b0 + 32].view(torch.int16)
        assert torch.equal(chunk, first.expand_as(chunk)), f"images {b0}.. differ from image 0"


def test_beyond_2gib(gpu):
    # Weights N(0, 0.02^2), the recipe of the C = 512 workloads (larger weights
    # put outputs near 16, where one bfloat16 rounding exceeds the 2e-2 bar).
    case = workloads.make_case(1, H, W, C, HEADS, M, (S,), "bf16", "v2", seed=88, w_std=0.02,
                               bias_std=0.05, tau="uniform")
    blk = case.blocks[0]
    dev = "cuda"
    x = case.x.to(dev).expand(B, H, W, C).contiguous()
    assert x.numel() * 2 >= 2 ** 31
    desc = gpu.make_desc(B, H, W, C, HEADS, M, S, "v2", torch.bfloat16)
    names = gpu.kernel_names(desc)
    _say(f"attention beyond 2 GiB: {names}")
    assert names[0] == "qkv_gemm_kernel" and names[2] == "proj_gemm_kernel"
    table = helpers.gpu_table(case, blk, dev)
    out = torch.full_like(x, float("nan"))
    y = gpu.wmsa_fwd(x, blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev),
                     blk.b_proj.to(dev), table, M, S, HEADS, "v2", tau=blk.tau.to(dev), out=out)
    torch.cuda.synchronize()
    _same_as_first(y)
    ref = helpers.run_oracle_block(case, blk, workloads.f64(case.x))
    helpers.assert_close(workloads.f64(y[0:1].cpu()), ref, "bf16", "attention, image 0")
    del out, y

    _say("block beyond 2 GiB (MLP hidden 2048)")
    extra = workloads.make_block_params(C, "bf16", 89, fc_std=0.02)
    gp = {"w_qkv": blk.w_qkv.to(dev), "b_qkv": blk.b_qkv.to(dev), "w_proj": blk.w_proj.to(dev),
          "b_proj": blk.b_proj.to(dev), "table": table, "tau": blk.tau.to(dev)}
    gp.update({k: v.to(dev) for k, v in extra.items()})
    out = torch.full_like(x, float("nan"))
    y = gpu.block_fwd(x, gp, M, S, HEADS, "v2", out=out)
    torch.cuda.synchronize()
    _same_as_first(y)
    op = {"w_qkv": workloads.f64(blk.w_qkv), "b_qkv": workloads.f64(blk.b_qkv),
          "w_proj": workloads.f64(blk.w_proj), "b_proj": workloads.f64(blk.b_proj),
          "table": helpers.oracle_table(case, blk), "tau": workloads.f64(blk.tau)}
    op.update({k: workloads.f64(v) for k, v in extra.items()})
    bref = sb.block_forward(workloads.f64(case.x), op, M, S, HEADS, "v2")
    helpers.assert_block_close(workloads.f64(y[0:1].cpu()), bref, "bf16", "block, image 0")
