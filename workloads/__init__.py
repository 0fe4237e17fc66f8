"""Seeded synthetic workloads for causal GQA attention with a QK-norm + RoPE prologue.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It holds the five workload shapes, a seeded input generator and the
fp32 -> bf16 input rounding; it contains none of the method's arithmetic (no
normalisation, rotation, softmax or contraction).

Shapes follow the pages' statement of the problem: attention tensors are laid out
as [batch * heads, seq_len, head_dim] (xtrain "Phase T15: GQA", Decision 1), with
K/V carrying num_kv_heads heads.  The tiny MHA shape is the tiny config of
"Phase T5: Tiny Transformer" (dim 32, 2 heads of 16); the dim768 shapes are the
bf16 training regime of "Phase T12: bf16 mixed precision"; the long-context GQA
shape uses the Qwen3 conventions of "Phase T9: Export to xserv" (theta = 1e6).

Input recipe (per workload k, seed k unless overridden):
    rng = numpy.random.default_rng(seed)
    draw float32 standard normals, in this order:
        xq (B, H, S, hd), xk (B, Hkv, S, hd), v (B, Hkv, S, hd), dout (B, H, S, hd),
        gamma_q (hd), gamma_k (hd)
    gamma = 1 for workloads whose gamma is "ones", else 1 + 0.1 * draw.
    bf16 workloads round xq, xk, v and dout to bf16 (round-to-nearest-even) before
    either side sees them; gamma stays fp32 (the fp32 master weight).
"""
from __future__ import annotations

import dataclasses
import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    seq_len: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str          # "f32" or "bf16": the io dtype of attention tensors
    gamma: str          # "ones" or "perturbed"
    eps: float
    theta: float

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def bh(self) -> int:
        return self.batch * self.num_heads

    @property
    def bkv(self) -> int:
        return self.batch * self.num_kv_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def causal_pairs(self) -> int:
        s = self.seq_len
        return s * (s + 1) // 2

    def attn_flops(self) -> dict:
        """Algorithmic flops: 4*hd per causal pair forward (QK^T, PV), 8*hd backward
        (dP, dV, dQ, dK); recompute is not counted."""
        units = self.causal_pairs() * self.bh
        return {"fwd": 4 * self.head_dim * units, "bwd": 8 * self.head_dim * units,
                "total": 12 * self.head_dim * units}


WORKLOADS = {
    1: Workload(1, "tiny_mha_f32", 1, 16, 2, 2, 16, "f32", "ones", 1e-5, 1e4),
    2: Workload(2, "gqa_g4_f32", 4, 256, 8, 2, 64, "f32", "perturbed", 1e-5, 1e4),
    3: Workload(3, "dim768_mha_bf16", 32, 1024, 12, 12, 64, "bf16", "ones", 1e-5, 1e4),
    4: Workload(4, "dim768_gqa_g3_bf16", 32, 1024, 12, 4, 64, "bf16", "perturbed", 1e-6, 1e4),
    5: Workload(5, "qwen3_long_gqa_g4_bf16", 1, 4096, 32, 8, 128, "bf16", "perturbed", 1e-6, 1e6),
    # The pages' own dim768 attention (24 heads of head_dim 32, sequence 256, per-rank batch
    # 32; xtrain "Phase T12", dim768 results table): an extra measured shape.
    6: Workload(6, "dim768_pages_hd32_bf16", 32, 256, 24, 24, 32, "bf16", "perturbed", 1e-5, 1e4),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even; returns the
    16-bit patterns as uint16.  NaN inputs are kept as a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16).astype(np.uint16) | 0x0040)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (RNE) -> float32."""
    return bf16_bits_to_f32(bf16_round_bits(x))


@dataclasses.dataclass
class Inputs:
    """Host float32 arrays (already bf16-representable for bf16 workloads)."""
    xq: np.ndarray       # [B*H, S, hd]
    xk: np.ndarray       # [B*Hkv, S, hd]
    v: np.ndarray        # [B*Hkv, S, hd]
    dout: np.ndarray     # [B*H, S, hd]
    gamma_q: np.ndarray  # [hd] fp32
    gamma_k: np.ndarray  # [hd] fp32


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    rng = np.random.default_rng(w.index if seed is None else seed)
    B, H, Hkv, S, hd = w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim
    xq = rng.standard_normal((B, H, S, hd), dtype=np.float32).reshape(B * H, S, hd)
    xk = rng.standard_normal((B, Hkv, S, hd), dtype=np.float32).reshape(B * Hkv, S, hd)
    v = rng.standard_normal((B, Hkv, S, hd), dtype=np.float32).reshape(B * Hkv, S, hd)
    dout = rng.standard_normal((B, H, S, hd), dtype=np.float32).reshape(B * H, S, hd)
    gq = rng.standard_normal(hd, dtype=np.float32)
    gk = rng.standard_normal(hd, dtype=np.float32)
    if w.gamma == "ones":
        gq = np.ones(hd, np.float32)
        gk = np.ones(hd, np.float32)
    else:
        gq = (1.0 + 0.1 * gq).astype(np.float32)
        gk = (1.0 + 0.1 * gk).astype(np.float32)
    if w.dtype == "bf16":
        xq, xk, v, dout = (bf16_round(a) for a in (xq, xk, v, dout))
    return Inputs(xq, xk, v, dout, gq, gk)


def small_ragged(dtype: str = "f32", head_dim: int = 64, seq_len: int = 77,
                 batch: int = 2, num_heads: int = 6, num_kv_heads: int = 2,
                 theta: float = 1e4, eps: float = 1e-5, gamma: str = "perturbed",
                 index: int = 101) -> Workload:
    """A small shape that spans several tiles and ends in a ragged tail."""
    return Workload(index, f"ragged_{dtype}_hd{head_dim}_s{seq_len}", batch, seq_len,
                    num_heads, num_kv_heads, head_dim, dtype, gamma, eps, theta)
