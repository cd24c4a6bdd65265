"""The C-ABI library loads, exports every symbol the header declares, and rejects
invalid calls on the host before launching anything.  CPU only: no call here
reaches a kernel launch."""
import ctypes
import os
import re

import pytest
import torch

import shifted_window_attention_roll_amd as swin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swin_wmsa.h")

OK, NULL, SHAPE, DTYPE, UNSUP, ALIAS, WS, ALIGN = 0, 1, 2, 3, 4, 5, 6, 7


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(swin.LIB_PATH):
        from shifted_window_attention_roll_amd import build
        build.build()
    return swin.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swin_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(swin._EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings(lib):
    assert lib.swin_abi_version() == 1
    for code in range(10):
        s = lib.swin_status_str(code).decode()
        assert s.startswith("SWIN_")
    assert lib.swin_status_str(99).decode() == "unknown swin_status"
    # no HIP error recorded yet on this thread: the runtime's text for success
    assert lib.swin_last_hip_error().decode()
    assert str(swin.SwinError(swin.SWIN_ERR_HIP)).startswith("SWIN_ERR_HIP: ")


def _desc(**kw):
    base = dict(B=2, H=56, W=56, C=96, heads=3, M=7, s=3, mode="v1", dtype=torch.float16)
    base.update(kw)
    return swin.make_desc(**base)


def test_workspace_size(lib):
    # small windows with <= 4 heads run as one fused kernel: no workspace
    assert swin.workspace_size(_desc()) == 0
    # window 16 with <= 4 heads and 16-bit I/O is fused too: one redo flag per
    # wave (2 per head) and window
    assert swin.workspace_size(_desc(H=64, W=64, C=128, heads=4, M=16, s=8)) == 2 * 16 * 8 * 4
    d = _desc(H=64, W=64, C=160, heads=5, M=8, s=4)
    T = 2 * 64 * 64
    assert swin.workspace_size(d) >= 4 * T * 160 * 2
    # QKV fused into the attention (window 16 or 24): only O (and the redo
    # flags) go through it
    d64 = _desc(H=64, W=64, C=192, heads=6, M=16, s=8)
    assert T * 192 * 2 <= swin.workspace_size(d64) < 2 * T * 192 * 2
    assert swin.workspace_size(_desc(B=0)) == 0
    assert swin.workspace_size(_desc(H=50)) == 0          # invalid -> 0
    # V2 with bf16 keeps q and k in float16: same byte count as bf16
    assert swin.workspace_size(swin.make_desc(2, 64, 64, 160, 5, 8, 4, "v2", torch.bfloat16)) == \
        swin.workspace_size(d)
    d32 = swin.make_desc(2, 64, 64, 128, 4, 16, 8, "v1", torch.float32)
    assert swin.workspace_size(d32) >= 4 * T * 128 * 4
    assert swin.workspace_size(_desc(C=512, heads=16)) >= 4 * 2 * 56 * 56 * 512 * 2


FAKE = 1 << 20  # host-side stand-in addresses; validation fails before any use


def _fwd(lib, d, x=FAKE, wq=FAKE * 2, wp=FAKE * 3, tab=FAKE * 4, tau=FAKE * 5, y=FAKE * 8,
         ws=FAKE * 16, ws_bytes=None, bq=None, bp=None):
    if ws_bytes is None:
        ws_bytes = lib.swin_wmsa_workspace_size(ctypes.byref(d))
    return lib.swin_wmsa_fwd(ctypes.byref(d), x, wq, bq, wp, bp, tab, tau, y, ws, ws_bytes, None)


def test_fwd_rejects_before_launch(lib):
    small = _desc(B=1, H=16, W=16, C=160, heads=5, M=16, s=3)  # needs a workspace
    assert _fwd(lib, _desc(H=50)) == SHAPE                   # H % M
    assert _fwd(lib, _desc(s=7)) == SHAPE                    # s >= M
    assert _fwd(lib, _desc(s=-1)) == SHAPE
    assert _fwd(lib, _desc(heads=5)) == SHAPE                # C % heads
    assert _fwd(lib, _desc(heads=1)) == UNSUP                # head dim 96
    assert _fwd(lib, _desc(M=28, s=0)) == UNSUP              # window beyond the LDS limit
    assert _fwd(lib, _desc(M=28, s=0, H=56)) == UNSUP
    assert _fwd(lib, _desc(mode=7)) == DTYPE
    assert _fwd(lib, _desc(dtype=9)) == DTYPE
    assert _fwd(lib, _desc(B=0)) == OK                        # empty: nothing to do
    assert _fwd(lib, small, x=None) == NULL
    assert _fwd(lib, small, tab=None) == NULL
    assert _fwd(lib, _desc(B=1, H=16, W=16, C=32, heads=1, M=16, s=3, mode="v2"), tau=None) == NULL
    assert _fwd(lib, small, ws_bytes=16) == WS
    assert _fwd(lib, small, y=FAKE + 64) == ALIAS             # y overlaps x
    assert _fwd(lib, small, ws=FAKE * 8 + 128) == ALIAS       # workspace overlaps y
    assert _fwd(lib, small, x=FAKE + 8) == ALIGN
    # A window holds at least 2 x 2 tokens.
    assert _fwd(lib, _desc(H=8, W=8, M=1, s=0)) == SHAPE
    # Every input is checked against the output and the workspace.
    v2 = _desc(B=1, H=16, W=16, C=160, heads=5, M=16, s=3, mode="v2")
    assert _fwd(lib, small, tab=FAKE * 8 + 64) == ALIAS       # bias table inside y
    assert _fwd(lib, small, tab=FAKE * 16 + 64) == ALIAS      # bias table inside the workspace
    assert _fwd(lib, v2, tau=FAKE * 8 + 4) == ALIAS           # tau inside y
    assert _fwd(lib, v2, tau=FAKE * 16 + 4) == ALIAS          # tau inside the workspace
    assert _fwd(lib, small, bq=FAKE * 8 + 32) == ALIAS        # b_qkv inside y
    assert _fwd(lib, small, bp=FAKE * 16 + 32) == ALIAS       # b_proj inside the workspace
    assert _fwd(lib, small, wq=FAKE * 16 + 32) == ALIAS       # w_qkv inside the workspace
    assert lib.swin_wmsa_fwd(None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, 0, None) == NULL


def test_index_maps_reject_before_launch(lib):
    f = lib.swin_partition_shift
    assert f(FAKE, FAKE * 4, 1, 14, 14, 8, 4, 1, 1, None) == SHAPE
    assert f(FAKE, FAKE * 4, 1, 14, 14, 8, 7, 7, 1, None) == SHAPE
    assert f(FAKE, FAKE * 4, 1, 14, 14, 8, 7, 3, 5, None) == DTYPE
    assert f(None, FAKE * 4, 1, 14, 14, 8, 7, 3, 1, None) == NULL
    assert f(FAKE, FAKE + 16, 1, 14, 14, 8, 7, 3, 1, None) == ALIAS
    assert f(FAKE + 2, FAKE * 4, 1, 14, 14, 8, 7, 3, 1, None) == ALIGN
    assert f(FAKE, FAKE * 4, 0, 14, 14, 8, 7, 3, 1, None) == OK
    assert f(FAKE, FAKE * 4, 1, 14, 14, 8, 1, 0, 1, None) == SHAPE  # M < 2
    assert lib.swin_reverse_unshift(FAKE, FAKE * 4, 1, 14, 12, 8, 7, 3, 1, None) == SHAPE


def test_cpb_rejects_before_launch(lib):
    f = lib.swin_cpb_table
    assert f(None, FAKE, FAKE, None, 512, 4, 16, 0.0, FAKE * 8, None) == NULL
    assert f(FAKE, FAKE * 2, FAKE * 3, None, 0, 4, 16, 0.0, FAKE * 8, None) == SHAPE
    assert f(FAKE, FAKE * 2, FAKE * 3, None, 512, 4, 33, 0.0, FAKE * 8, None) == SHAPE
    assert f(FAKE, FAKE * 2, FAKE * 3, None, 512, 4, 16, 0.0, FAKE + 64, None) == ALIAS
    assert f(FAKE, FAKE * 2, FAKE * 3, None, 512, 4, 1, 0.0, FAKE * 8, None) == SHAPE  # M < 2


def test_binding_refuses_cpu_tensors(lib):
    x = torch.zeros(1, 7, 7, 32)
    with pytest.raises(ValueError):
        swin.partition_shift(x, 7, 3)


def test_kernel_names_and_timed_rejects(lib):
    d = _desc(H=64, W=64, C=128, heads=4, M=16, s=8)
    tiled = ["qkv_tiled_kernel", "tiled_attn_kernel", "proj_tiled_kernel"]
    three = ["qkv_gemm_kernel", "window_attn_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(d) == ["fused_w16_kernel", "fused_w16_redo_kernel"]
    assert swin.kernel_names(_desc(H=64, W=64, C=160, heads=5, M=8, s=4)) == [
        "qkv_gemm_kernel", "tiled_attn_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(_desc(H=64, W=64, C=160, heads=5, M=16, s=8)) == [
        "fused_qkv_attn_kernel", "fused_qkv_attn_redo_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=24, s=12, C=512, heads=16,
                                   dtype=torch.bfloat16)) == ["fused_qkv_attn_kernel",
                                                              "fused_qkv_attn_redo_kernel",
                                                              "proj_tiled_kernel"]
    assert swin.kernel_names(_desc(H=64, W=64, M=16, s=8, C=192, heads=6)) == [
        "fused_qkv_attn_kernel", "fused_qkv_attn_redo_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=24, s=12, C=96, heads=3,
                                   dtype=torch.bfloat16)) == ["fused_qkv_attn_kernel",
                                                              "fused_qkv_attn_redo_kernel",
                                                              "proj_gemm_kernel"]
    # window 16 with x of 2^31 elements or more: not the single fused kernel
    assert swin.kernel_names(_desc(B=4096, H=64, W=64, C=128, heads=4, M=16, s=8,
                                   dtype=torch.bfloat16))[0] != "fused_w16_kernel"
    # x of 2 GiB or more: the three-kernel plan
    assert swin.kernel_names(_desc(B=232, H=96, W=96, M=24, s=12, C=512, heads=16,
                                   dtype=torch.bfloat16))[0] == "qkv_gemm_kernel"
    assert swin.kernel_names(_desc(H=48, W=48, M=8, s=4, C=512, heads=16,
                                   dtype=torch.bfloat16)) == tiled
    assert swin.kernel_names(_desc(H=64, W=64, M=16, s=8, C=128, heads=4,
                                   dtype=torch.float32)) == three
    assert swin.kernel_names(_desc()) == ["fused_w8_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=8, s=4, C=64, heads=2,
                                   dtype=torch.bfloat16, mode="v2")) == ["fused_w8_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=8, s=4, C=128, heads=4,
                                   dtype=torch.bfloat16, mode="v2")) == ["fused_w8_kernel"]
    assert swin.kernel_names(_desc(dtype=torch.float32)) == ["fused_window_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=6, s=3)) == ["fused_window_kernel"]
    assert swin.kernel_names(_desc(C=512, heads=16)) == ["qkv_tiled_kernel", "w8_attn_kernel",
                                                          "proj_tiled_kernel"]
    assert swin.kernel_names(_desc(C=512, heads=16, dtype=torch.float32)) == [
        "qkv_gemm_kernel", "window_attn_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(_desc(H=14, W=14, C=160, heads=5)) == [
        "qkv_gemm_kernel", "w8_attn_kernel", "proj_gemm_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=12, s=6, C=128, heads=4)) == three
    assert swin.kernel_names(_desc(H=48, W=48, M=12, s=6, C=256, heads=8)) == [
        "qkv_tiled_kernel", "window_attn_kernel", "proj_tiled_kernel"]
    assert swin.kernel_names(_desc(H=48, W=48, M=16, s=6, C=96, heads=3)) == [
        "fused_w16_kernel", "fused_w16_redo_kernel"]
    assert lib.swin_wmsa_kernel_count(ctypes.byref(_desc(H=50))) == 0
    assert lib.swin_wmsa_kernel_name(ctypes.byref(d), 3) is None
    small = _desc(B=1, H=16, W=16, C=160, heads=5, M=16, s=3)  # needs a workspace
    ws = lib.swin_wmsa_workspace_size(ctypes.byref(small))
    ev = (ctypes.c_void_p * 4)(FAKE * 64, FAKE * 65, FAKE * 66, FAKE * 67)
    args = (ctypes.byref(small), FAKE, FAKE * 2, None, FAKE * 3, None, FAKE * 4, None, FAKE * 8,
            FAKE * 16, ws, None)
    assert lib.swin_wmsa_fwd_timed(*args, None, 4) == NULL
    assert lib.swin_wmsa_fwd_timed(*args, ev, 3) == SHAPE
    ev_null = (ctypes.c_void_p * 4)(FAKE * 64, None, FAKE * 66, FAKE * 67)
    assert lib.swin_wmsa_fwd_timed(*args, ev_null, 4) == NULL


def _block(lib, d, x=FAKE, y=FAKE * 8, ws=FAKE * 64, ws_bytes=None, **over):
    if ws_bytes is None:
        ws_bytes = lib.swin_block_workspace_size(ctypes.byref(d))
    names = [f[0] for f in swin.BlockParams._fields_]
    vals = {n: FAKE * (100 + i) for i, n in enumerate(names)}
    vals.update(over)
    bp = swin.BlockParams(*[vals[n] for n in names])
    return lib.swin_block_fwd(ctypes.byref(d), x, ctypes.byref(bp), y, ws, ws_bytes, None)


def test_block_workspace_size(lib):
    d = swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, "v1", torch.float16)
    T = 2 * 56 * 56
    # three [T, C] intermediates and one [T, 4C], 16-bit (the attention needs none here)
    assert lib.swin_block_workspace_size(ctypes.byref(d)) >= 3 * T * 96 * 2 + T * 384 * 2
    d2 = swin.make_block_desc(2, 64, 64, 160, 5, 16, 8, "v1", torch.bfloat16)
    assert lib.swin_block_workspace_size(ctypes.byref(d2)) >= \
        swin.workspace_size(d2.attn) + 3 * 2 * 64 * 64 * 160 * 2
    assert lib.swin_block_workspace_size(ctypes.byref(
        swin.make_block_desc(2, 50, 56, 96, 3, 7, 3))) == 0                   # H % M
    assert lib.swin_block_workspace_size(ctypes.byref(
        swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, hidden=100))) == 0       # hidden % 32


def test_block_rejects_before_launch(lib):
    d = swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, "v1", torch.float16)
    assert _block(lib, swin.make_block_desc(0, 56, 56, 96, 3, 7, 3)) == OK    # empty batch
    assert _block(lib, swin.make_block_desc(2, 50, 56, 96, 3, 7, 3)) == SHAPE
    assert _block(lib, swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, hidden=48)) == SHAPE
    assert _block(lib, swin.make_block_desc(1, 14, 14, 1024, 32, 7, 3)) == UNSUP  # C > 512
    assert _block(lib, d, x=None) == NULL
    assert _block(lib, d, ln2_g=None) == NULL
    assert _block(lib, d, fc1_w=None) == NULL
    assert _block(lib, swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, "v2"), tau=None) == NULL
    assert _block(lib, d, ws_bytes=64) == WS
    assert _block(lib, d, y=FAKE + 64) == ALIAS                              # y overlaps x
    # every parameter is checked against y and the workspace
    for name in [f[0] for f in swin.BlockParams._fields_]:
        if name == "tau":
            continue
        assert _block(lib, d, **{name: FAKE * 8 + 16}) == ALIAS, name          # inside y
        assert _block(lib, d, **{name: FAKE * 64 + 16}) == ALIAS, name         # inside the ws
    dv2 = swin.make_block_desc(2, 56, 56, 96, 3, 7, 3, "v2", torch.float16)
    assert _block(lib, dv2, tau=FAKE * 8 + 4) == ALIAS
    assert _block(lib, d, x=FAKE + 8) == ALIGN
    assert lib.swin_block_fwd(None, FAKE, None, FAKE, FAKE, 0, None) == NULL


def _bwd(lib, d, x=FAKE, wq=FAKE * 2, wp=FAKE * 3, tab=FAKE * 4, tau=FAKE * 5, dy=FAKE * 6,
         grads=None, ws=FAKE * 64, ws_bytes=None, **g):
    if ws_bytes is None:
        ws_bytes = lib.swin_wmsa_bwd_workspace_size(ctypes.byref(d))
    fields = dict(dx=FAKE * 8, dw_qkv=FAKE * 9, db_qkv=FAKE * 10, dw_proj=FAKE * 11,
                  db_proj=FAKE * 12, dtable=FAKE * 13, dtau=FAKE * 14)
    fields.update(g)
    gr = swin.Grads(*[fields[n] for n in ("dx", "dw_qkv", "db_qkv", "dw_proj", "db_proj",
                                          "dtable", "dtau")])
    return lib.swin_wmsa_bwd(ctypes.byref(d), x, wq, None, wp, tab, tau, dy,
                             None if grads == "null" else ctypes.byref(gr), ws, ws_bytes, None)


def test_bwd_workspace_size(lib):
    d = _desc(B=1)
    T, C = 56 * 56, 96
    parts = [T * C * 2] * 3 + [T * 3 * C * 4, T * C * 4, T * C * 4, T * 3 * C * 4]
    assert swin.bwd_workspace_size(d) == sum((p + 255) // 256 * 256 for p in parts)
    assert swin.bwd_workspace_size(_desc(B=0)) == 0
    assert swin.bwd_workspace_size(_desc(H=48, W=48, M=24, s=0, dtype=torch.bfloat16)) > 0
    assert swin.bwd_workspace_size(_desc(H=48, W=48, M=24, s=0, dtype=torch.float32)) > 0
    assert swin.bwd_workspace_size(_desc(H=50, W=50, M=25, s=0, dtype=torch.bfloat16)) == 0
    assert swin.bwd_workspace_size(_desc(heads=1)) == 0


def test_bwd_rejects_before_launch(lib):
    d = _desc(B=1)
    assert _bwd(lib, _desc(B=1, H=50, W=50, M=25, s=0, dtype=torch.bfloat16)) == UNSUP
    assert _bwd(lib, _desc(B=1, heads=5)) == SHAPE
    assert _bwd(lib, d, wq=None) == NULL
    assert _bwd(lib, d, dy=None) == NULL
    assert _bwd(lib, d, grads="null") == NULL
    assert _bwd(lib, d, dtable=None) == NULL
    assert _bwd(lib, _desc(B=1, mode="v2"), dtau=None) == NULL
    assert _bwd(lib, d, ws_bytes=16) == WS
    assert _bwd(lib, d, dx=FAKE + 64) == ALIAS                # dx overlaps x
    assert _bwd(lib, d, dw_proj=FAKE * 9 + 4) == ALIAS        # two outputs overlap
    assert _bwd(lib, d, dtable=FAKE * 64 + 256) == ALIAS      # output inside the workspace
    assert _bwd(lib, d, x=FAKE + 8) == ALIGN
    assert _bwd(lib, d, ws=FAKE * 64 + 8) == ALIGN
    assert lib.swin_wmsa_bwd(None, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, 0,
                             None) == NULL


def test_cpb_bwd_rejects_before_launch(lib):
    assert lib.swin_cpb_bwd_workspace_size(512, 16, 24) == ((47 * 47 * 16 * 4 + 255) // 256) * 256
    assert lib.swin_cpb_bwd_workspace_size(512, 65, 24) == 0
    F = FAKE

    def call(**kw):
        a = dict(w1=F, b1=F * 2, w2=F * 3, b2=F * 4, hidden=512, heads=16, M=24, dt=F * 5,
                 dw1=F * 8, db1=F * 9, dw2=F * 10, db2=F * 11, ws=F * 12, wsb=1 << 20)
        a.update(kw)
        return lib.swin_cpb_bwd(a["w1"], a["b1"], a["w2"], a["b2"], a["hidden"], a["heads"],
                                a["M"], 0.0, a["dt"], a["dw1"], a["db1"], a["dw2"], a["db2"],
                                a["ws"], a["wsb"], None)
    assert call(w1=None) == NULL
    assert call(ws=None) == NULL
    assert call(heads=0) == SHAPE
    assert call(M=33) == SHAPE
    assert call(wsb=16) == WS
    assert call(dw2=F * 3 + 4) == ALIAS          # output over an input
    assert call(db1=F * 8 + 4) == ALIAS          # two outputs overlap


def test_fp8_rejects_before_launch(lib):
    q = lib.swin_fp8_quantize
    assert q(FAKE, 9, 4, 64, FAKE * 4, FAKE * 8, None) == DTYPE
    assert q(FAKE, 2, 4, 0, FAKE * 4, FAKE * 8, None) == SHAPE
    assert q(FAKE, 2, 0, 64, FAKE * 4, FAKE * 8, None) == OK          # empty
    assert q(None, 2, 4, 64, FAKE * 4, FAKE * 8, None) == NULL
    assert q(FAKE, 2, 4, 64, FAKE + 16, FAKE * 8, None) == ALIAS      # codes inside x
    assert q(FAKE + 8, 2, 4, 64, FAKE * 4, FAKE * 8, None) == ALIGN
    f = lib.swin_fp8_linear
    a = dict(a=FAKE, sa=FAKE * 2, w=FAKE * 3, sw=FAKE * 4, b=None, bdt=2, y=FAKE * 8, ydt=2,
             rows=16, N=64, K=128)

    def call(**kw):
        v = dict(a)
        v.update(kw)
        return f(v["a"], v["sa"], v["w"], v["sw"], v["b"], v["bdt"], v["y"], v["ydt"], v["rows"],
                 v["N"], v["K"], None)
    assert call(ydt=9) == DTYPE
    assert call(K=48) == SHAPE                   # K % 32
    assert call(rows=0) == OK
    assert call(sw=None) == NULL
    assert call(y=FAKE * 3 + 64) == ALIAS        # y over the weight codes
    assert call(b=FAKE * 8 + 16) == ALIAS        # bias inside y
    assert call(w=FAKE * 3 + 4) == ALIGN


def test_sparse24_rejects_before_launch(lib):
    c = lib.swin_sparse24_compress
    assert c(FAKE, 0, 64, 64, FAKE * 4, FAKE * 8, None) == DTYPE     # float32
    assert c(FAKE, 2, 64, 66, FAKE * 4, FAKE * 8, None) == SHAPE     # K % 4
    assert c(FAKE, 2, 0, 64, FAKE * 4, FAKE * 8, None) == OK
    assert c(FAKE, 2, 64, 64, FAKE + 64, FAKE * 8, None) == ALIAS    # values inside w
    f = lib.swin_sparse24_linear
    a = dict(x=FAKE, v=FAKE * 2, c=FAKE * 3, b=None, y=FAKE * 8, dt=2, rows=16, N=64, K=128)

    def call(**kw):
        v = dict(a)
        v.update(kw)
        return f(v["x"], v["v"], v["c"], v["b"], v["y"], v["dt"], v["rows"], v["N"], v["K"], None)
    assert call(dt=0) == DTYPE
    assert call(K=96) == SHAPE                   # K % 64
    assert call(rows=0) == OK
    assert call(c=None) == NULL
    assert call(y=FAKE * 2 + 64) == ALIAS        # y over the kept values
    assert call(c=FAKE * 3 + 4) == ALIGN         # positions are read 16 bytes at a time
    assert call(c=FAKE * 3 + 8) == ALIGN


# Kernels the forward can enqueue, per plan: the parity cases with the tau clip
# and the descriptor overrides (test_gpu_parity.PLAN_CASES) must reach each.
PLAN_KERNELS = {"fused_w8_kernel", "fused_window_kernel", "fused_w16_kernel", "fused_w16_redo_kernel",
                "fused_qkv_attn_kernel", "fused_qkv_attn_redo_kernel",
                "tiled_attn_kernel", "w8_attn_kernel", "window_attn_kernel",
                "qkv_tiled_kernel", "qkv_gemm_kernel", "proj_tiled_kernel", "proj_gemm_kernel"}


def test_override_cases_cover_every_plan(lib):
    from test_gpu_parity import PLAN_CASES
    seen = set()
    for (B, H, W, C, heads, M, s, dtype) in PLAN_CASES:
        dt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
        for mode in ("v1", "v2"):
            seen.update(swin.kernel_names(swin.make_desc(B, H, W, C, heads, M, s, mode, dt)))
    assert seen == PLAN_KERNELS


def test_noalloc_rejects_before_launch(lib):
    f = lib.swin_wmsa_fwd_noalloc
    big = _desc(B=64, H=384, W=384, C=512, heads=16, M=24, s=12, dtype=torch.bfloat16)
    assert lib.swin_wmsa_workspace_size(ctypes.byref(big)) > swin.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), FAKE, FAKE * 2, None, FAKE * 3, None, FAKE * 4, None, FAKE * 8,
             None) == 9                                          # SWIN_ERR_SCRATCH
    assert f(ctypes.byref(_desc(H=50)), FAKE, FAKE * 2, None, FAKE * 3, None, FAKE * 4, None,
             FAKE * 8, None) == SHAPE
    assert f(ctypes.byref(_desc(B=0)), FAKE, FAKE * 2, None, FAKE * 3, None, FAKE * 4, None,
             FAKE * 8, None) == OK
    assert f(None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None) == NULL
