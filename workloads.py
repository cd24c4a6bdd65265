"""Seeded synthetic inputs for the shifted-window attention block forward.

This module only draws random tensors and names the workload shapes.  It holds
none of the method's arithmetic (no shift, no partition, no attention), so that
both the HIP path and the CPU oracle can take their inputs from here without
sharing any computation.

Shapes follow Swin stage shapes (Swin-T stage 1, Swin-B stage 3, SwinV2-B
stage 1 and a SwinV2-G-like 1536x1536 stage 1 with patch 4); the pages measure on
ImageNet / COCO / ADE20K images, which these seeded tensors stand in for.

Recipe (every workload):
  * numpy ``Generator(PCG64(SeedSequence(seed)))``; the seed is spawned into
    child streams in the fixed order x, W_qkv, b_qkv, W_proj, b_proj,
    bias-table-or-CPB-MLP (W1, b1, W2, b2), tau, repeated per block.
  * values drawn in float32, then rounded to the I/O dtype by round-to-nearest-
    even (torch ``.to``); the rounded values are what both sides consume.
  * x ~ N(0, 1); W_qkv, W_proj ~ N(0, 0.02^2); b_qkv, b_proj = 0;
    V1 relative-position table ~ N(0, 0.02^2) (float32);
    V2 CPB MLP: W1 ~ N(0, 1), b1 ~ N(0, 1), W2 ~ N(0, 1/512), b2 = 0 (float32);
    V2 tau: 0.1 for every head (SwinV2-B) or U(0.01, 0.1) per head (SwinV2-G-like).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}

# Workloads: name -> shape.  ``shifts`` lists one entry per block forward in one
# pass (the Swin-T full-batch workload alternates a plain and a shifted block).
WORKLOADS: Dict[str, dict] = {
    # Swin-T stage 1, one image: small enough for the oracle to run in seconds.
    "swin_t_stage1_b1_fp32": dict(B=1, H=56, W=56, C=96, heads=3, M=7, shifts=(3,),
                                  dtype="fp32", mode="v1", tau=None, seed=1000),
    # Swin-T stage 1, full batch of 64: W-MSA (shift 0) then SW-MSA (shift 3).
    "swin_t_stage1_b64_fp16": dict(B=64, H=56, W=56, C=96, heads=3, M=7, shifts=(0, 3),
                                   dtype="fp16", mode="v1", tau=None, seed=1001),
    # Swin-B stage 3: 14x14 tokens, 4 windows per image, heavy masking.
    "swin_b_stage3_b64_bf16": dict(B=64, H=14, W=14, C=512, heads=16, M=7, shifts=(3,),
                                   dtype="bf16", mode="v1", tau=None, seed=1002),
    # SwinV2-B stage 1 with window 16 and scaled cosine attention.
    "swinv2_b_stage1_w16_bf16": dict(B=32, H=64, W=64, C=128, heads=4, M=16, shifts=(8,),
                                     dtype="bf16", mode="v2", tau="const0.1", seed=1003),
    # SwinV2-G-like stage 1 at 1536x1536 (patch 4 -> 384x384 tokens), window 24.
    "swinv2_g_stage1_384_w24_bf16": dict(B=1, H=384, W=384, C=512, heads=16, M=24,
                                         shifts=(12,), dtype="bf16", mode="v2",
                                         tau="uniform", seed=1004),
}


@dataclasses.dataclass
class BlockParams:
    """Parameters of one attention block; tensors are CPU torch tensors."""
    s: int
    w_qkv: torch.Tensor            # [3C, C], I/O dtype
    b_qkv: torch.Tensor            # [3C], I/O dtype
    w_proj: torch.Tensor           # [C, C], I/O dtype
    b_proj: torch.Tensor           # [C], I/O dtype
    table: Optional[torch.Tensor]  # V1: [(2M-1)^2, heads] float32
    cpb_w1: Optional[torch.Tensor]  # V2: [hidden, 2] float32
    cpb_b1: Optional[torch.Tensor]  # V2: [hidden]
    cpb_w2: Optional[torch.Tensor]  # V2: [heads, hidden]
    cpb_b2: Optional[torch.Tensor]  # V2: [heads]
    tau: Optional[torch.Tensor]    # V2: [heads] float32, raw (unclipped)


@dataclasses.dataclass
class Case:
    B: int
    H: int
    W: int
    C: int
    heads: int
    M: int
    dtype: str
    mode: str
    x: torch.Tensor                # [B, H, W, C], I/O dtype
    blocks: List[BlockParams]

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.W


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _to(a: np.ndarray, dtype: str) -> torch.Tensor:
    # torch's float32 -> fp16/bf16 conversion rounds to nearest even.
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DTYPES[dtype])


def make_case(B: int, H: int, W: int, C: int, heads: int, M: int,
              shifts: Sequence[int], dtype: str, mode: str, seed: int,
              tau: Optional[str] = None, x_std: float = 1.0, w_std: float = 0.02,
              bias_std: float = 0.0, table_std: float = 0.02, cpb_hidden: int = 512,
              tau_value: float = 0.1) -> Case:
    """Draw one seeded case.  ``bias_std`` > 0 gives non-zero linear biases
    (used by tests to exercise the bias path; the workloads use zeros)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype}")
    if mode not in ("v1", "v2"):
        raise ValueError(f"unknown mode {mode}")
    n_streams = 1 + 10 * len(shifts)
    children = np.random.SeedSequence(seed).spawn(n_streams)
    gens = [np.random.Generator(np.random.PCG64(c)) for c in children]
    x = _to(_normal(gens[0], (B, H, W, C), x_std), dtype)
    nrel = (2 * M - 1) ** 2
    blocks = []
    for bi, s in enumerate(shifts):
        g = gens[1 + 10 * bi: 1 + 10 * (bi + 1)]
        w_qkv = _to(_normal(g[0], (3 * C, C), w_std), dtype)
        b_qkv = _to(_normal(g[1], (3 * C,), bias_std) if bias_std > 0
                    else np.zeros(3 * C, np.float32), dtype)
        w_proj = _to(_normal(g[2], (C, C), w_std), dtype)
        b_proj = _to(_normal(g[3], (C,), bias_std) if bias_std > 0
                     else np.zeros(C, np.float32), dtype)
        table = cw1 = cb1 = cw2 = cb2 = tau_t = None
        if mode == "v1":
            table = torch.from_numpy(_normal(g[4], (nrel, heads), table_std))
        else:
            cw1 = torch.from_numpy(_normal(g[5], (cpb_hidden, 2), 1.0))
            cb1 = torch.from_numpy(_normal(g[6], (cpb_hidden,), 1.0))
            cw2 = torch.from_numpy(_normal(g[7], (heads, cpb_hidden), (1.0 / cpb_hidden) ** 0.5))
            cb2 = torch.zeros(heads, dtype=torch.float32)
            if tau is None or tau == "const0.1":
                tau_t = torch.full((heads,), np.float32(tau_value), dtype=torch.float32)
            elif tau == "uniform":
                tau_t = torch.from_numpy(g[8].uniform(0.01, 0.1, size=heads).astype(np.float32))
            else:
                raise ValueError(f"unknown tau recipe {tau}")
        blocks.append(BlockParams(s=s, w_qkv=w_qkv, b_qkv=b_qkv, w_proj=w_proj,
                                  b_proj=b_proj, table=table, cpb_w1=cw1, cpb_b1=cb1,
                                  cpb_w2=cw2, cpb_b2=cb2, tau=tau_t))
    return Case(B=B, H=H, W=W, C=C, heads=heads, M=M, dtype=dtype, mode=mode, x=x,
                blocks=blocks)


def make_block_params(C: int, dtype: str, seed: int, hidden: Optional[int] = None,
                      fc_std: float = 0.1, ln_std: float = 0.1) -> Dict[str, torch.Tensor]:
    """Seeded parameters of the rest of a full block (the LayerNorms and the MLP),
    rounded to ``dtype``: ln*_g ~ N(1, ln_std), ln*_b ~ N(0, ln_std), fc1 [hidden, C]
    and fc2 [C, hidden] ~ N(0, fc_std), their biases ~ N(0, fc_std / 2); hidden
    defaults to 4C."""
    hidden = 4 * C if hidden is None else hidden
    g = [np.random.Generator(np.random.PCG64(c))
         for c in np.random.SeedSequence(seed).spawn(8)]
    return {
        "ln1_g": _to(1.0 + _normal(g[0], (C,), ln_std), dtype),
        "ln1_b": _to(_normal(g[1], (C,), ln_std), dtype),
        "ln2_g": _to(1.0 + _normal(g[2], (C,), ln_std), dtype),
        "ln2_b": _to(_normal(g[3], (C,), ln_std), dtype),
        "fc1_w": _to(_normal(g[4], (hidden, C), fc_std), dtype),
        "fc1_b": _to(_normal(g[5], (hidden,), fc_std / 2), dtype),
        "fc2_w": _to(_normal(g[6], (C, hidden), fc_std), dtype),
        "fc2_b": _to(_normal(g[7], (C,), fc_std / 2), dtype),
    }


def make_upstream_grad(shape, dtype: str, seed: int, std: float = 1.0) -> torch.Tensor:
    """Seeded N(0, std) upstream gradient dL/dy of ``shape``, rounded to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return _to(_normal(rng, tuple(shape), std), dtype)


def make_workload(name: str, B: Optional[int] = None) -> Case:
    """The named workload; ``B`` overrides the batch (same per-image recipe)."""
    w = dict(WORKLOADS[name])
    seed = w.pop("seed")
    if B is not None:
        w["B"] = B
    return make_case(seed=seed, **w)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU tensor (every fp16/bf16/fp32 value is exact in fp64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def random_bits(shape, dtype: str, seed: int) -> torch.Tensor:
    """Random bit patterns (NaN payloads and subnormals included) viewed as ``dtype``,
    for tests of kernels that only move data."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    if dtype == "fp32":
        a = rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)
        return torch.from_numpy(a.view(np.int32)).view(torch.float32)
    a = rng.integers(0, 2 ** 16, size=shape, dtype=np.uint32).astype(np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(DTYPES[dtype])
