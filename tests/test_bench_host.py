"""Host-side logic of bench.py (no GPU): which sources a kernel's traffic
counters are tied to."""
import os

import bench

CSRC = os.path.join(bench.ROOT, "shifted_window_attention_roll_amd", "csrc")


def _closure(kernel):
    return {os.path.basename(p) for p in
            bench._source_closure(CSRC, [bench.KERNEL_SOURCE[kernel], "api.hip"])}


def test_every_kernel_source_exists():
    for k, f in bench.KERNEL_SOURCE.items():
        assert os.path.exists(os.path.join(CSRC, f)), k


def test_digest_follows_includes():
    w8 = _closure("fused_w8_kernel")
    assert {"fused_w8.hip", "w8_core.hpp", "kv_frag.hpp", "common.hpp", "api.hip"} <= w8
    assert "attn_core.hpp" not in w8 and "fused_w16.hip" not in w8
    assert "attn_core.hpp" in _closure("tiled_attn_kernel")
    assert bench.source_digest("fused_w8_kernel") != bench.source_digest("tiled_attn_kernel")
    assert bench.source_digest("qkv_tiled_kernel") == bench.source_digest("proj_tiled_kernel")


def test_cpu_sample_windows_cover_the_masked_edge():
    # one 384 x 384 image, window 24: 256 windows; the sample spans the grid,
    # first and last (masked) window included
    w = bench._sample_windows(1, 384, 384, 24, 32)
    assert w[0] == 0 and w[-1] == 255 and len(w) == 32
    assert bench._sample_windows(1, 48, 48, 24, 99) == [0, 1, 2, 3]


def test_headline_is_the_largest_single_gpu_workload():
    import workloads
    flops = {n: bench.flops_per_token(w["C"], w["M"] ** 2) * w["B"] * w["H"] * w["W"] *
             len(w["shifts"]) for n, w in workloads.WORKLOADS.items()}
    assert bench.MAIN == max(flops, key=flops.get)


def test_traffic_record_is_used_only_on_matching_sources(tmp_path, monkeypatch):
    # A record taken on other kernel sources reads as unmeasured (None); one
    # whose digest matches gives its bytes per launch.
    import json
    k, w = "fused_qkv_attn_kernel", "swinv2_g_stage1_384_w24_bf16"
    digest = bench.source_digest(k)
    (tmp_path / "profiles").mkdir()
    rec = {"entries": {f"{w}:{k}": {"bytes_per_launch": 123.0, "source_digest": digest},
                       f"{w}:proj_tiled_kernel": {"bytes_per_launch": 7.0,
                                                  "source_digest": "0" * 16}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: digest)
    assert bench.measured_traffic(k, w) == 123.0
    assert bench.measured_traffic("proj_tiled_kernel", w) is None
    assert bench.measured_traffic(k, "swin_b_stage3_b64_bf16") is None
