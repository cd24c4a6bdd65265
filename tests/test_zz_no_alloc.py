"""swin_wmsa_fwd_noalloc (the library's fixed device scratch as the workspace)
against swin_wmsa_fwd with a caller workspace: bit-identical outputs (the same
kernels on the same inputs), on two calls in a row, the second smaller, for
plans that use the workspace (three kernels) and one that needs none."""
import sys

import pytest
import torch

import workloads

import helpers

pytestmark = pytest.mark.gpu


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


def _both(gpu, case, dev="cuda"):
    blk = case.blocks[0]
    x = case.x.to(dev)
    args = (x, blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev), blk.b_proj.to(dev),
            helpers.gpu_table(case, blk, dev), case.M, blk.s, case.heads, case.mode)
    tau = None if blk.tau is None else blk.tau.to(dev)
    ref = gpu.wmsa_fwd(*args, tau=tau)
    out = torch.full_like(x, float("nan"))
    got = gpu.wmsa_fwd_noalloc(*args, tau=tau, out=out)
    torch.cuda.synchronize()
    return got, ref


# (first call, second call with a smaller input), per plan
PAIRS = [
    # window 24, C = 512: QKV GEMM / attention / projection through the scratch
    ((2, 48, 48, 512, 16, 24, 12, "bf16", "v2"), (1, 24, 48, 512, 16, 24, 12, "bf16", "v2")),
    # window 7 with 16 heads (Swin-B stage 3 shape at batch 8, then 3)
    ((8, 14, 14, 512, 16, 7, 3, "bf16", "v1"), (3, 14, 14, 512, 16, 7, 3, "bf16", "v1")),
    # general three kernels, float32
    ((2, 32, 32, 64, 2, 16, 8, "fp32", "v2"), (1, 16, 32, 64, 2, 16, 8, "fp32", "v2")),
    # a fused plan (no scratch needed)
    ((4, 56, 56, 96, 3, 7, 3, "fp16", "v1"), (1, 28, 28, 96, 3, 7, 3, "fp16", "v1")),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry(gpu, first, second):
    for i, (B, H, W, C, heads, M, s, dtype, mode) in enumerate((first, second)):
        _say(f"noalloc call {i}: B={B} H={H} W={W} C={C} heads={heads} M={M} s={s} {dtype} {mode}")
        desc = gpu.make_desc(B, H, W, C, heads, M, s, mode, workloads.DTYPES[dtype])
        assert gpu.workspace_size(desc) <= gpu.NOALLOC_SCRATCH_BYTES
        case = workloads.make_case(B, H, W, C, heads, M, (s,), dtype, mode, seed=900 + i + C,
                                   w_std=0.02, bias_std=0.05, tau="uniform")
        got, ref = _both(gpu, case)
        assert torch.isfinite(got.float()).all()
        it = torch.int32 if dtype == "fp32" else torch.int16
        assert torch.equal(got.view(it), ref.view(it))


def test_noalloc_rejects_beyond_scratch(gpu):
    B, H, W, C, heads, M, s = 4, 384, 384, 512, 16, 24, 12
    desc = gpu.make_desc(B, H, W, C, heads, M, s, "v2", torch.bfloat16)
    assert gpu.workspace_size(desc) > gpu.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, H, W, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * C, C), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros((C, C), dtype=torch.bfloat16, device="cuda")
    tab = torch.zeros(((2 * M - 1) ** 2, heads), device="cuda")
    tau = torch.ones(heads, device="cuda")
    with pytest.raises(gpu.SwinError):
        gpu.wmsa_fwd_noalloc(x, w, None, wp, None, tab, M, s, heads, "v2", tau=tau)
