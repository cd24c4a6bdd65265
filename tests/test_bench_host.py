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
