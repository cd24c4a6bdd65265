"""GPU parity of the FP8 (E4M3) linear layers (swin_fp8_quantize,
swin_fp8_linear through the C ABI) against oracle/swin_fp8.py.

Codes and scales are integer / float32 decisions that both sides take in
float32: compared bit for bit.  The product: every 8-bit product is exact in
float32, the K-term sums are not, and y is rounded once to its dtype, so per
element |gpu - oracle| <= u |oracle| + 2 K 2^-24 (|a| |w|^T)[r, n] sa[r] sw[n]
(u = 0 float32, 2^-11 float16, 2^-8 bfloat16), derived, written in the test.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import swin_fp8 as f8

pytestmark = pytest.mark.gpu

U = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shifted_window_attention_roll_amd as swin
    swin.load_library()
    return swin


def _matrix(rows, K, dtype, seed, std=1.0):
    x = workloads.make_upstream_grad((rows, K), dtype, seed, std)
    # Wide dynamic range per row: some rows tiny, some with a large outlier,
    # one all-zero row, a few exact zeros.
    x = x.float()
    r = np.random.default_rng(seed)
    x[:, :] *= torch.from_numpy(2.0 ** r.integers(-12, 6, (rows, 1))).float()
    if rows > 3:
        x[1, :] = 0.0
        x[2, 5 % K] = 300.0
        x[3, ::7] = 0.0
    return x.to(workloads.DTYPES[dtype])


@pytest.mark.parametrize("rows,K,dtype", [(37, 96, "fp32"), (64, 512, "bf16"), (5, 2048, "fp16"),
                                          (130, 40, "bf16"), (1, 1, "fp32")])
def test_quantize_bit_exact(gpu, rows, K, dtype):
    _say(f"fp8 quantize rows={rows} K={K} {dtype}")
    x = _matrix(rows, K, dtype, rows + K)
    codes, scales = gpu.fp8_quantize(x.cuda())
    torch.cuda.synchronize()
    qo, so = f8.quantize_rows(x.float().numpy())
    np.testing.assert_array_equal(codes.cpu().numpy(), qo)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), so.view(np.uint32))


def _check_linear(got, qa, sa, qw, sw, bias, out_dtype, rows_idx=None):
    ref = f8.linear_fp8(qa, sa, qw, sw, bias)
    absdot = (np.abs(f8.e4m3_decode(qa)) @ np.abs(f8.e4m3_decode(qw)).T) * \
        np.asarray(sa, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]
    K = qa.shape[1]
    bound = U[out_dtype] * np.abs(ref) + 2 * K * 2.0 ** -24 * absdot + 1e-30
    err = np.abs(got - ref)
    _say(f"  max err {err.max():.3g}, max err / bound {float((err / bound).max()):.3g}")
    assert np.all(err <= bound), float((err - bound).max())


@pytest.mark.parametrize("rows,N,K,in_dtype,out_dtype", [
    (100, 96, 96, "fp16", torch.float16),       # ragged rows and columns
    (64, 288, 96, "bf16", torch.bfloat16),
    (33, 64, 512, "fp32", torch.float32),
    (256, 1536, 512, "bf16", torch.bfloat16),   # QKV of a C = 512 stage
    (70, 512, 2048, "bf16", torch.float32),     # long K
    # the persistent tiled product (K in 512 .. 2048, N % 128 == 0): several
    # 256-row tiles per workgroup, a ragged last one
    (1000, 384, 1024, "fp16", torch.float16),
    (777, 256, 1536, "bf16", torch.float32),
])
def test_linear(gpu, rows, N, K, in_dtype, out_dtype):
    _say(f"fp8 linear rows={rows} N={N} K={K} {in_dtype} -> {out_dtype}")
    x = workloads.make_upstream_grad((rows, K), in_dtype, rows * 3 + K)
    w = workloads.make_upstream_grad((N, K), in_dtype, N * 5 + K, std=0.02)
    b = workloads.make_upstream_grad((N,), in_dtype, N + 11, std=0.1)
    qa, sa = gpu.fp8_quantize(x.cuda())
    qw, sw = gpu.fp8_quantize(w.cuda())
    y = gpu.fp8_linear(qa, sa, qw, sw, b.cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    qao, sao = f8.quantize_rows(x.float().numpy())
    qwo, swo = f8.quantize_rows(w.float().numpy())
    _check_linear(workloads.f64(y.cpu()), qao, sao, qwo, swo, workloads.f64(b), out_dtype)


@pytest.mark.parametrize("name", ["swin_b_stage3_b64_bf16", "swinv2_g_stage1_384_w24_bf16"])
def test_linear_workload_qkv_sampled(gpu, name):
    # The QKV projection of the workload's full token count (window order does
    # not matter to a per-token layer); 64 sampled rows compared.
    case = workloads.make_workload(name)
    blk = case.blocks[-1]
    T, C = case.tokens, case.C
    _say(f"fp8 linear {name}: {T} x {3 * C} x {C}")
    x = case.x.reshape(T, C)
    qa, sa = gpu.fp8_quantize(x.cuda())
    qw, sw = gpu.fp8_quantize(blk.w_qkv.cuda())
    y = gpu.fp8_linear(qa, sa, qw, sw, blk.b_qkv.cuda(), out_dtype=x.dtype)
    torch.cuda.synchronize()
    rows = np.random.default_rng(9).choice(T, 64, replace=False)
    qao, sao = f8.quantize_rows(x[rows].float().numpy())
    qwo, swo = f8.quantize_rows(blk.w_qkv.float().numpy())
    _check_linear(workloads.f64(y[rows].cpu()), qao, sao, qwo, swo, workloads.f64(blk.b_qkv),
                  x.dtype)


def test_linear_without_bias(gpu):
    _say("fp8 linear without bias")
    x = workloads.make_upstream_grad((40, 256), "bf16", 5)
    w = workloads.make_upstream_grad((128, 256), "bf16", 6, std=0.02)
    qa, sa = gpu.fp8_quantize(x.cuda())
    qw, sw = gpu.fp8_quantize(w.cuda())
    y = gpu.fp8_linear(qa, sa, qw, sw, None, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    qao, sao = f8.quantize_rows(x.float().numpy())
    qwo, swo = f8.quantize_rows(w.float().numpy())
    _check_linear(workloads.f64(y.cpu()), qao, sao, qwo, swo, None, torch.bfloat16)
