"""Seeded synthetic inputs and the workload table.

This module holds no arithmetic of the retention method: it only draws random tensors and
lists the workload shapes, decays and seeds. Both the tests (for the oracle and the GPU path)
and the benchmark draw their inputs from here.

Input recipe: q, k and v are i.i.d. N(0, 1) / sqrt(d_k), drawn in that order from a torch
generator seeded with the workload's seed, then rounded to the workload's input dtype.
The per-head decays are gamma_h = 1 - 2^(-5 - h) for h = 0 .. H-1 unless a workload lists its
own; every such value is exact in fp32 and fp64.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def multiscale_gammas(H: int):
    """gamma_h = 1 - 2^(-5-h), h = 0..H-1 (0-based head index), as Python floats."""
    return [1.0 - 2.0 ** (-5 - h) for h in range(H)]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    dk: int
    dv: int
    dtype: str            # input dtype: "f32" or "bf16"
    chunks: Tuple[int, ...]
    seed: int
    gammas: Optional[Tuple[float, ...]] = None
    groupnorm: bool = False
    eps: float = 1e-5
    out_dtype: str = "f32"
    note: str = ""

    def gamma_list(self):
        return list(self.gammas) if self.gammas is not None else multiscale_gammas(self.H)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("retention_b1_h2_n256_d64_f32", 1, 2, 256, 64, 64, "f32", (64,), seed=1, gammas=(0.9, 0.99),
                 note="tiny: parallel, recurrent and chunkwise forms must agree"),
        Workload("retention_b4_h8_n2048_d64_bf16", 4, 8, 2048, 64, 64, "bf16", (128,), seed=2),
        Workload("retention_b1_h16_n8192_dk256_dv512_bf16_gn", 1, 16, 8192, 256, 512, "bf16", (128,), seed=3,
                 groupnorm=True, eps=1e-5, out_dtype="bf16", note="6.7B-layer-shaped chunkwise with GroupNorm"),
        Workload("decode_b128_h16_dk256_dv512", 128, 16, 1, 256, 512, "bf16", (128,), seed=4,
                 note="one recurrent step on fp32 states from a chunkwise prefill of 8192 tokens"),
        Workload("retention_b1_h16_n65536_dk256_dv512_bf16", 1, 16, 65536, 256, 512, "bf16", (64, 128, 256, 512),
                 seed=5, note="long context, chunk sweep, final state checked"),
    ]
}

DECODE_PREFILL_TOKENS = 8192


def make_qkv(B: int, H: int, N: int, dk: int, dv: int, dtype: str, seed: int, device="cpu"):
    """q, k, v ~ N(0,1)/sqrt(dk), drawn in that order from a generator seeded with `seed`."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    s = 1.0 / (dk ** 0.5)
    out = []
    for d in (dk, dk, dv):
        x = torch.randn((B, H, N, d), generator=gen, device=device, dtype=torch.float32) * s
        out.append(x.to(DTYPES[dtype]))
    return tuple(out)


def make_workload_qkv(w: Workload, device="cpu", N: Optional[int] = None):
    return make_qkv(w.B, w.H, w.N if N is None else N, w.dk, w.dv, w.dtype, w.seed, device=device)


def make_state(B: int, H: int, dk: int, dv: int, seed: int, scale: float = 1.0, device="cpu"):
    """A random fp32 state [B,H,dk,dv] ~ scale * N(0,1), for tests of state_in / decode."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn((B, H, dk, dv), generator=gen, device=device, dtype=torch.float32) * scale
