"""One step of the hot path over preallocated device buffers.

A step is the whole path once: RoPE cos/sin cache and QK-norm + RoPE on K (one launch),
attention forward (out, lse) with QK-norm + RoPE of Q fused into it, then the backward (delta, dq, dk/dv with
the group sum, prologue backward for Q and K, dgamma reductions).  Buffers are allocated once at
construction with torch (plumbing only); every step runs only libxattn kernels, on one
stream, with no allocation.
"""
from __future__ import annotations

import torch

from . import (Dims, make_dims, segments, xattn_bwd, xattn_bwd_workspace_bytes,
               xattn_fwd_qnorm, xattn_qknorm_rope_fwd_table)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


class AttentionStep:
    """doc_lengths: optional document lengths packed along the sequence axis (summing to
    seq_len, the same packing for every batch row): block-causal mask and RoPE positions
    restarting in every document."""

    def __init__(self, batch, seq_len, num_heads, num_kv_heads, head_dim, dtype, eps, theta,
                 device="cuda", doc_lengths=None):
        self.B, self.S, self.H, self.Hkv, self.hd = batch, seq_len, num_heads, num_kv_heads, head_dim
        self.eps, self.theta = float(eps), float(theta)
        self.dtype = _TORCH_DTYPE[dtype] if isinstance(dtype, str) else dtype
        dev = torch.device(device)
        f32 = torch.float32
        qshape = (batch * num_heads, seq_len, head_dim)
        kshape = (batch * num_kv_heads, seq_len, head_dim)
        e = lambda shape, dt=self.dtype: torch.empty(shape, dtype=dt, device=dev)
        # inputs
        self.xq, self.xk, self.v, self.dout = e(qshape), e(kshape), e(kshape), e(qshape)
        self.gamma_q, self.gamma_k = e(head_dim, f32), e(head_dim, f32)
        # forward products
        self.cos, self.sin = e((seq_len, head_dim // 2), f32), e((seq_len, head_dim // 2), f32)
        self.yq, self.yk = e(qshape), e(kshape)
        self.rstd_q = e(batch * num_heads * seq_len, f32)
        self.rstd_k = e(batch * num_kv_heads * seq_len, f32)
        self.out, self.lse = e(qshape), e(batch * num_heads * seq_len, f32)
        # backward products (w.r.t. the raw inputs)
        self.dxq, self.dxk, self.dv = e(qshape), e(kshape), e(kshape)
        self.dgamma_q, self.dgamma_k = e(head_dim, f32), e(head_dim, f32)
        self.seg = None
        if doc_lengths is not None:
            if sum(int(n) for n in doc_lengths) != seq_len:
                raise ValueError("doc_lengths must sum to seq_len")
            self.seg = segments(doc_lengths, dev)  # (seg_lo, seg_hi, positions)
        self.dims: Dims = make_dims(self.yq, num_heads, num_kv_heads,
                                    None if self.seg is None else self.seg[:2])
        self.workspace = torch.empty(max(16, xattn_bwd_workspace_bytes(self.dims, True)),
                                     dtype=torch.uint8, device=dev)
        self.prologue = dict(xq=self.xq, xk=self.xk, gamma_q=self.gamma_q, gamma_k=self.gamma_k,
                             rstd_q=self.rstd_q, rstd_k=self.rstd_k, cos_tab=self.cos,
                             sin_tab=self.sin, dgamma_q=self.dgamma_q, dgamma_k=self.dgamma_k)

    def load(self, xq, xk, v, dout, gamma_q, gamma_k):
        """Copy host (numpy / torch) inputs into the device buffers."""
        for dst, src in ((self.xq, xq), (self.xk, xk), (self.v, v), (self.dout, dout),
                         (self.gamma_q, gamma_q), (self.gamma_k, gamma_k)):
            t = torch.as_tensor(src)
            dst.copy_(t.reshape(dst.shape).to(dst.dtype))
        return self

    def forward(self, stream=None):
        S, hd = self.S, self.hd
        # RoPE table (positions restart per document when there are documents) and the K
        # prologue in one launch
        xattn_qknorm_rope_fwd_table(self.xk, self.gamma_k,
                                    None if self.seg is None else self.seg[2], self.theta,
                                    self.cos, self.sin, self.yk, self.rstd_k, self.B * self.Hkv,
                                    S, hd, self.eps, stream)
        xattn_fwd_qnorm(self.dims, self.xq, self.gamma_q, self.cos, self.sin, self.eps, self.yq,
                        self.rstd_q, self.yk, self.v, self.out, self.lse, stream)

    def backward(self, stream=None):
        xattn_bwd(self.dims, self.yq, self.yk, self.v, self.out, self.lse, self.dout, self.dxq,
                  self.dxk, self.dv, self.prologue, self.workspace, stream)

    def run(self, stream=None):
        self.forward(stream)
        self.backward(stream)

    def results(self):
        """Host float64 numpy copies of every output of the step."""
        names = ["yq", "yk", "rstd_q", "rstd_k", "out", "lse", "dxq", "dxk", "dv", "dgamma_q",
                 "dgamma_k", "cos", "sin"]
        return {n: getattr(self, n).detach().to(torch.float64).cpu().numpy() for n in names}
