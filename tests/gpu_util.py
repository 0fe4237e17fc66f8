"""Shared helpers for the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import causal_gqa_attention_amd as X
import oracle
import workloads as W
from causal_gqa_attention_amd.step import AttentionStep

# Norm-wise max relative error bound per io dtype: max|x - r| / max|r| per tensor.
TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(x, r):
    """Norm-wise relative error max|x - r| / max|r|.  Where the reference is identically
    zero (e.g. dq and dk of a single-token sequence) the bound applies to the absolute
    error instead (all inputs are O(1))."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        return 0.0
    den = np.abs(r).max()
    return float(np.abs(x - r).max() / (den if den > 0 else 1.0))


def p99_err(x, r):
    """Elementwise diagnostic: the 99th percentile of |x - r| / (|r| + 1e-3 max|r|).  It is
    printed next to the norm-wise error (a wrong low-magnitude region shows here first);
    the pass bar is the norm-wise one."""
    x = np.asarray(x, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    if x.size == 0:
        return 0.0
    den = np.abs(r) + 1e-3 * np.abs(r).max()
    den = np.where(den > 0, den, 1.0)
    return float(np.percentile(np.abs(x - r) / den, 99))


def assert_close(name, x, r, tol):
    """Norm-wise bar on one tensor (non-finite values fail); prints the norm-wise error and
    the elementwise p99 diagnostic, returns the norm-wise error."""
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    e = rel_err(x, r)
    print(f"  {name}: norm-wise {e:.2e}  p99 elementwise {p99_err(x, r):.2e}")
    assert e <= tol, f"{name}: norm-wise rel err {e:.3e} > {tol:.1e}"
    return e


def dev(a, dtype):
    return torch.as_tensor(np.ascontiguousarray(a)).to("cuda").to(TDT[dtype])


def host(t):
    return t.detach().to(torch.float64).cpu().numpy()


# Every output buffer of a step; poison() fills them with NaN before a run, so an element
# that no kernel writes fails the finiteness check of assert_close.
STEP_OUTPUTS = ("yq", "yk", "rstd_q", "rstd_k", "out", "lse", "dxq", "dxk", "dv", "dgamma_q",
                "dgamma_k", "cos", "sin")


def poison(step: AttentionStep):
    for n in STEP_OUTPUTS:
        getattr(step, n).fill_(float("nan"))
    torch.cuda.synchronize()


def run_step(w: W.Workload, x: W.Inputs, doc_lengths=None) -> dict:
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta, doc_lengths=doc_lengths)
    step.load(x.xq, x.xk, x.v, x.dout, x.gamma_q, x.gamma_k)
    poison(step)
    step.run()
    torch.cuda.synchronize()
    return step.results()


def attention_only(w: W.Workload, q, k, v, dout):
    """GPU attention forward and backward (no prologue) on the given host arrays; every
    output buffer starts as NaN."""
    tq, tk, tv, td = (dev(a, w.dtype) for a in (q, k, v, dout))
    nan = float("nan")
    out, dq = torch.full_like(tq, nan), torch.full_like(tq, nan)
    dk, dv = torch.full_like(tk, nan), torch.full_like(tv, nan)
    lse = torch.full((tq.shape[0] * tq.shape[1],), nan, dtype=torch.float32, device=tq.device)
    dims = X.make_dims(tq, w.num_heads, w.num_kv_heads)
    X.xattn_fwd(dims, tq, tk, tv, out, lse)
    ws = torch.empty(max(16, X.xattn_bwd_workspace_bytes(dims, False)), dtype=torch.uint8,
                     device=tq.device)
    X.xattn_bwd(dims, tq, tk, tv, out, lse, td, dq, dk, dv, None, ws)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in dict(out=out, lse=lse, dq=dq, dk=dk, dv=dv).items()}


def seeded_attention_inputs(w: W.Workload, seed: int):
    """q, k, v, dout drawn like the workload recipe (bf16-rounded for bf16)."""
    rng = np.random.default_rng(seed)
    B, H, Hkv, S, hd = w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim
    q = rng.standard_normal((B * H, S, hd), dtype=np.float32)
    k = rng.standard_normal((B * Hkv, S, hd), dtype=np.float32)
    v = rng.standard_normal((B * Hkv, S, hd), dtype=np.float32)
    do = rng.standard_normal((B * H, S, hd), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v, do = (W.bf16_round(a) for a in (q, k, v, do))
    return q, k, v, do


def sampled_kv_heads(w: W.Workload, n=2):
    """A few B*Hkv indices spread over the tensor (first, last, middle)."""
    cand = [0, w.bkv - 1, w.bkv // 2, w.bkv // 3]
    out = []
    for c in cand:
        if c not in out:
            out.append(c)
    return out[:n]


def q_heads_of(w: W.Workload, kv):
    b, kvh = divmod(kv, w.num_kv_heads)
    return [b * w.num_heads + kvh * w.group + r for r in range(w.group)]
