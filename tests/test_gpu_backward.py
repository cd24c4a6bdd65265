"""GPU parity of the sub-layer backward (swin_wmsa_bwd through the C ABI)
against the float64 backward oracle on the same seeded inputs.

Bar (derived; every step runs in float32 on inputs that the oracle takes
exactly): per gradient tensor, max |gpu - oracle| <= 1e-4 x max |oracle| and
relative L2 <= 1e-4; the 16-bit dx is also rounded once on output, which adds
u |oracle| per element (u = 2^-8 bfloat16, 2^-11 float16).  dtau is one sum of
B nW N^2 products per head whose terms cancel (by a factor near 2e4 at window
24): each term carries float32 rounding, so its bar adds 2 x 2^-24 x the sum of
|terms| (the oracle's dtau_abs) instead of a relative-L2 test.
"""
import sys

import numpy as np
import pytest
import torch

import helpers
import workloads
from oracle import swin_backward as sbw

pytestmark = pytest.mark.gpu

TOL = 1e-4
ULP = {"fp32": 0.0, "fp16": 2.0 ** -11, "bf16": 2.0 ** -8}


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


def _run(swin, B, H, W, C, heads, M, s, dtype, mode, seed, tau=None):
    case = workloads.make_case(B, H, W, C, heads, M, (s,), dtype, mode, seed=seed, w_std=0.08,
                               bias_std=0.1, table_std=0.3, tau="uniform")
    blk = case.blocks[0]
    if tau is not None:
        blk.tau = torch.tensor(tau, dtype=torch.float32)
    dy = workloads.make_upstream_grad(case.x.shape, dtype, seed + 1)
    dev = "cuda"
    g = swin.wmsa_bwd(case.x.to(dev), blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev),
                      helpers.gpu_table(case, blk, dev), dy.to(dev), M, s, heads, mode,
                      tau=None if blk.tau is None else blk.tau.to(dev))
    torch.cuda.synchronize()
    ref = sbw.wmsa_backward(workloads.f64(case.x), workloads.f64(blk.w_qkv),
                            workloads.f64(blk.b_qkv), workloads.f64(blk.w_proj),
                            workloads.f64(blk.b_proj), helpers.oracle_table(case, blk), M, s,
                            heads, workloads.f64(dy), mode,
                            tau=None if blk.tau is None else workloads.f64(blk.tau))
    return g, ref


def _assert_grads(g, ref, dtype, mode, what):
    keys = ["dx", "dw_qkv", "db_qkv", "dw_proj", "db_proj", "dtable"] + (["dtau"] if mode == "v2"
                                                                         else [])
    for k in keys:
        got = workloads.f64(g[k].cpu())
        r = ref[k]
        assert got.shape == r.shape, (what, k, got.shape, r.shape)
        assert np.isfinite(got).all(), (what, k)
        scale = max(float(np.abs(r).max()), 1e-30)
        err = np.abs(got - r)
        bound = TOL * scale + (ULP[dtype] * np.abs(r) if k == "dx" else 0.0)
        if k == "dtau":
            bound = bound + 2.0 * 2.0 ** -24 * ref["dtau_abs"]
        worst = float((err - bound).max())
        rel = float(np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30))
        _say(f"  {what} {k}: max err {err.max():.3g} (scale {scale:.3g}), rel-L2 {rel:.3g}")
        assert worst <= 0, (what, k, float(err.max()), scale)
        if k != "dtau":
            assert rel <= TOL + 2 * ULP[dtype] * (k == "dx"), (what, k, rel)


CASES = [
    # B, H, W, C, heads, M, s, dtype, mode
    (2, 14, 14, 64, 2, 7, 3, "fp32", "v1"),
    (1, 14, 21, 96, 3, 7, 0, "fp32", "v1"),     # no shift, H != W
    (1, 16, 16, 64, 2, 8, 4, "fp32", "v2"),
    (1, 32, 32, 64, 2, 16, 8, "fp32", "v1"),    # window 16 (256-thread kernel)
    (1, 32, 48, 32, 1, 16, 5, "fp32", "v2"),    # window 16, odd split
    (2, 14, 14, 96, 3, 7, 3, "bf16", "v1"),
    (1, 16, 24, 128, 4, 8, 1, "fp16", "v2"),
    (1, 32, 32, 64, 2, 16, 8, "bf16", "v2"),
    (1, 12, 12, 32, 1, 4, 2, "fp32", "v1"),     # window 4
    (1, 7, 7, 32, 1, 7, 3, "fp32", "v2"),       # window = image, shifted
    (1, 20, 30, 64, 2, 10, 5, "fp32", "v1"),    # window 10: 100 tokens padded to 128
    (2, 12, 12, 64, 2, 3, 1, "fp32", "v2"),     # window 3: 9 tokens padded to 32
    (1, 48, 48, 64, 2, 24, 12, "fp32", "v1"),   # window 24: two 288-row chunks per phase
    (1, 48, 24, 32, 1, 24, 7, "bf16", "v2"),    # window 24, odd split, 16-bit I/O
    (1, 34, 17, 64, 2, 17, 8, "fp32", "v2"),    # window 17: 289 tokens, ragged last tile
    (1, 40, 20, 32, 1, 20, 0, "fp16", "v1"),    # window 20 unshifted: 400 tokens of 576
]


@pytest.mark.parametrize("B,H,W,C,heads,M,s,dtype,mode", CASES)
def test_backward_small(gpu, B, H, W, C, heads, M, s, dtype, mode):
    what = f"bwd B={B} H={H} W={W} C={C} heads={heads} M={M} s={s} {dtype} {mode}"
    _say(what)
    g, ref = _run(gpu, B, H, W, C, heads, M, s, dtype, mode, seed=1000 + H + C + s)
    _assert_grads(g, ref, dtype, mode, what)


def test_backward_clamped_tau(gpu):
    # Head 1's tau under the clip: its gradient is exactly zero, head 0's is not.
    _say("bwd clamped tau")
    g, ref = _run(gpu, 1, 16, 16, 64, 2, 8, 4, "fp32", "v2", seed=77, tau=[0.2, 0.004])
    _assert_grads(g, ref, "fp32", "v2", "clamped tau")
    dt = g["dtau"].cpu()
    assert float(dt[1]) == 0.0 and float(dt[0]) != 0.0


def test_backward_empty_batch(gpu):
    _say("bwd empty batch")
    swin = gpu
    dev = "cuda"
    x = torch.empty(0, 14, 14, 64, device=dev)
    grads = {"dx": torch.empty_like(x),
             "dw_qkv": torch.full((192, 64), 7.0, device=dev),
             "db_qkv": torch.full((192,), 7.0, device=dev),
             "dw_proj": torch.full((64, 64), 7.0, device=dev),
             "db_proj": torch.full((64,), 7.0, device=dev),
             "dtable": torch.full((169, 2), 7.0, device=dev)}
    w = torch.zeros(192, 64, device=dev)
    swin.wmsa_bwd(x, w, None, torch.zeros(64, 64, device=dev), torch.zeros(169, 2, device=dev),
                  torch.empty_like(x), 7, 3, 2, "v1", grads=grads)
    torch.cuda.synchronize()
    for k, v in grads.items():
        if k != "dx":
            assert float(v.abs().max()) == 0.0, k


def test_backward_swin_t_stage1_batch16(gpu):
    # The benchmark's shape (Swin-T stage 1, 56 x 56, C = 96, 3 heads, window 7,
    # shift 3, float16) at batch 16: every token of every window compared.
    what = "bwd Swin-T stage 1 B=16 fp16"
    _say(what)
    g, ref = _run(gpu, 16, 56, 56, 96, 3, 7, 3, "fp16", "v1", seed=4242)
    _assert_grads(g, ref, "fp16", "v1", what)


def test_backward_deterministic_except_atomics(gpu):
    # Two calls: dx (no atomics) bit-identical; the atomically summed gradients
    # agree to float32 reassociation.
    _say("bwd repeat")
    a, _ = _run(gpu, 2, 14, 14, 64, 2, 7, 3, "fp32", "v1", seed=5)
    b, _ = _run(gpu, 2, 14, 14, 64, 2, 7, 3, "fp32", "v1", seed=5)
    assert torch.equal(a["dx"], b["dx"])
    for k in ("dw_qkv", "dw_proj", "dtable"):
        scale = float(a[k].abs().max())
        torch.testing.assert_close(a[k], b[k], rtol=0, atol=1e-6 * scale)


@pytest.mark.parametrize("M,hidden,heads", [(8, 512, 4), (16, 256, 3), (24, 512, 16), (3, 64, 1)])
def test_cpb_backward(gpu, M, hidden, heads):
    # Meta-network backward against the oracle's, for a seeded table gradient.
    _say(f"cpb bwd M={M} hidden={hidden} heads={heads}")
    case = workloads.make_case(1, M, M, 32 * heads, heads, M, (0,), "bf16", "v2", seed=M + hidden,
                               cpb_hidden=hidden)
    blk = case.blocks[0]
    dt = workloads.make_upstream_grad(((2 * M - 1) ** 2, heads), "fp32", M * 7)
    dev = "cuda"
    got = gpu.cpb_bwd(blk.cpb_w1.to(dev), blk.cpb_b1.to(dev), blk.cpb_w2.to(dev),
                      blk.cpb_b2.to(dev), M, dt.to(dev))
    torch.cuda.synchronize()
    ref = sbw.cpb_backward(workloads.f64(blk.cpb_w1), workloads.f64(blk.cpb_b1),
                           workloads.f64(blk.cpb_w2), workloads.f64(blk.cpb_b2), M,
                           workloads.f64(dt))
    for k in ("dw1", "db1", "dw2", "db2"):
        g = workloads.f64(got[k].cpu())
        r = ref[k]
        scale = max(float(np.abs(r).max()), 1e-30)
        err = float(np.abs(g - r).max())
        _say(f"  {k}: max err {err:.3g} (scale {scale:.3g})")
        assert err <= TOL * scale, (k, err, scale)


def test_backward_large_bias(gpu):
    # A bias table with std 4 (logit spreads of tens): the exact row maxima keep
    # every exponential finite; gradients still at the bar.
    _say("bwd large bias")
    case = workloads.make_case(1, 16, 16, 64, 2, 8, (4,), "fp32", "v1", seed=31, w_std=0.08,
                               bias_std=0.1, table_std=4.0)
    blk = case.blocks[0]
    dy = workloads.make_upstream_grad(case.x.shape, "fp32", 32)
    g = gpu.wmsa_bwd(case.x.cuda(), blk.w_qkv.cuda(), blk.b_qkv.cuda(), blk.w_proj.cuda(),
                     blk.table.cuda(), dy.cuda(), 8, 4, 2, "v1")
    torch.cuda.synchronize()
    ref = sbw.wmsa_backward(workloads.f64(case.x), workloads.f64(blk.w_qkv),
                            workloads.f64(blk.b_qkv), workloads.f64(blk.w_proj),
                            workloads.f64(blk.b_proj), workloads.f64(blk.table), 8, 4, 2,
                            workloads.f64(dy), "v1")
    _assert_grads(g, ref, "fp32", "v1", "large bias")


def test_backward_full_size_sampled_windows(gpu):
    # SwinV2-G stage 1 (384 x 384, C 512, 16 heads, window 24, shift 12,
    # bfloat16) as the bench times it: dx of five windows (first, interior,
    # last-column, last-row and corner; the last three masked) against the
    # oracle run on those windows alone, every element of dx finite, and the
    # closed forms that hold at any size: db_proj is the sum of dy, and each
    # head's table gradient sums to zero.
    from oracle import swin_oracle as so
    name = "swinv2_g_stage1_384_w24_bf16"
    _say(f"bwd full size {name}")
    swin = gpu
    case = workloads.make_workload(name)
    blk = case.blocks[-1]
    M, s, heads, C = case.M, blk.s, case.heads, case.C
    dy = workloads.make_upstream_grad(case.x.shape, case.dtype, 3)
    dev = "cuda"
    g = swin.wmsa_bwd(case.x.to(dev), blk.w_qkv.to(dev), blk.b_qkv.to(dev), blk.w_proj.to(dev),
                      helpers.gpu_table(case, blk, dev), dy.to(dev), M, s, heads, case.mode,
                      tau=None if blk.tau is None else blk.tau.to(dev))
    torch.cuda.synchronize()
    dx = g["dx"].float().cpu()
    assert torch.isfinite(dx).all()
    nwx = case.W // M
    windows = [0, 5 * nwx + 7, 9 * nwx + nwx - 1, (case.H // M - 1) * nwx + 3,
               (case.H // M) * nwx - 1]
    ref = sbw.wmsa_backward(workloads.f64(case.x), workloads.f64(blk.w_qkv),
                            workloads.f64(blk.b_qkv), workloads.f64(blk.w_proj),
                            workloads.f64(blk.b_proj), helpers.oracle_table(case, blk), M, s,
                            heads, workloads.f64(dy), case.mode,
                            tau=None if blk.tau is None else workloads.f64(blk.tau),
                            windows=windows)
    src = so.window_token_source(case.B, case.H, case.W, M, s)[windows]   # [5, N]
    got = workloads.f64(dx).reshape(-1, C)[src]
    r = ref["dxw"]
    scale = float(np.abs(r).max())
    err = np.abs(got - r)
    bound = TOL * scale + ULP[case.dtype] * np.abs(r)
    rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
    _say(f"  dx on {len(windows)} windows: max err {err.max():.3g} (scale {scale:.3g}), "
         f"rel-L2 {rel:.3g}")
    assert float((err - bound).max()) <= 0
    assert rel <= TOL + 2 * ULP[case.dtype]
    dbp = g["db_proj"].cpu().double().numpy()
    dbp_ref = workloads.f64(dy).reshape(-1, C).sum(axis=0)
    assert np.abs(dbp - dbp_ref).max() <= TOL * np.abs(dbp_ref).max()
    dt = g["dtable"].cpu().double().numpy()
    assert (np.abs(dt.sum(axis=0)) <= TOL * np.abs(dt).sum(axis=0)).all()
