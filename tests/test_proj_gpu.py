"""Parity of the projections around attention (Mint documentation 5.3.1-5.3.2: q = x Wq +
bq, ..., Concat(heads) Wo + bo; "Phase T5" head split / merge; "Phase T12": GEMMs in the io
dtype with fp32 accumulation, fp32 weight and bias gradients) with the float64 oracle,
forward and backward, and of the whole attention block (projections + prologue + attention
+ output projection) with the oracle's composition."""
import numpy as np
import pytest
import torch

import causal_gqa_attention_amd as X
import oracle
import workloads as W
from gpu_util import TOL, TDT, assert_close, dev, host, note

pytestmark = pytest.mark.gpu

# (dtype, B, S, H, Hkv, hd, d, bias)
SHAPES = [
    ("f32", 2, 37, 4, 2, 64, 96, True),
    ("bf16", 2, 37, 4, 2, 64, 96, True),
    ("bf16", 1, 300, 8, 2, 128, 256, False),
    ("f32", 1, 16, 2, 2, 16, 32, True),
    ("bf16", 32, 1024, 12, 4, 64, 768, True),   # dim768 GQA shape (split-K weight grads)
    ("bf16", 1, 4096, 32, 8, 128, 4096, True),  # Qwen3-shaped heads, d = 4096
    ("bf16", 3, 50, 6, 2, 32, 200, True),       # ragged rows, columns and K in every GEMM
    ("bf16", 2, 33, 4, 4, 16, 40, False),       # hd 16: 4-column output runs inside a head
    ("bf16", 3, 128, 4, 2, 64, 200, True),      # head-major operands read in place, 3 sequences
    ("bf16", 2, 192, 2, 1, 128, 136, True),     # ... at hd 128, ragged model dim
    ("f32", 3, 50, 6, 2, 32, 200, False),
]
IDS = [f"{s[0]}_B{s[1]}_S{s[2]}_H{s[3]}_kv{s[4]}_hd{s[5]}_d{s[6]}_{'bias' if s[7] else 'nobias'}"
       for s in SHAPES]


def _inputs(dt, B, S, H, Hkv, hd, d, bias, seed):
    rng = np.random.default_rng(seed)
    f32 = np.float32
    r = (lambda a: W.bf16_round(a)) if dt == "bf16" else (lambda a: a)
    x = r(rng.standard_normal((B * S, d), dtype=f32))
    ws = [r((rng.standard_normal((d, n), dtype=f32) / np.sqrt(d)).astype(f32))
          for n in (H * hd, Hkv * hd, Hkv * hd)]
    wo = r((rng.standard_normal((H * hd, d), dtype=f32) / np.sqrt(H * hd)).astype(f32))
    bs = [(0.1 * rng.standard_normal(n, dtype=f32)).astype(f32) if bias else None
          for n in (H * hd, Hkv * hd, Hkv * hd, d)]
    return x, ws, wo, bs


def _proj(dt, B, S, H, Hkv, hd, ws, wo, bs):
    t = [dev(w, dt) for w in ws] + [dev(wo, dt)]
    b = [dev(v, "f32") if v is not None else None for v in bs]
    return X.Projection(B, S, H, Hkv, hd, *t, *b)


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_projections_forward_and_backward_match_oracle(shape):
    dt, B, S, H, Hkv, hd, d, bias = shape
    x, ws, wo, bs = _inputs(dt, B, S, H, Hkv, hd, d, bias, 600 + B + S + d)
    note(f"projections {shape}")
    pr = _proj(dt, B, S, H, Hkv, hd, ws, wo, bs)
    rng = np.random.default_rng(7)
    r = (lambda a: W.bf16_round(a)) if dt == "bf16" else (lambda a: a)
    out = r(rng.standard_normal((B * H, S, hd), dtype=np.float32))
    dy = r(rng.standard_normal((B * S, d), dtype=np.float32))
    gq = r(rng.standard_normal((B * H, S, hd), dtype=np.float32))
    gk = r(rng.standard_normal((B * Hkv, S, hd), dtype=np.float32))
    gv = r(rng.standard_normal((B * Hkv, S, hd), dtype=np.float32))
    tx = dev(x, dt)
    xq, xk, v = pr.qkv_fwd(tx)
    y = pr.out_fwd(dev(out, dt))
    dout, dwo, dbo = pr.out_bwd(dev(out, dt), dev(dy, dt), with_bias=bias)
    dx, dws, dbs = pr.qkv_bwd(tx, dev(gq, dt), dev(gk, dt), dev(gv, dt), with_bias=bias)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(x, *ws, *bs[:3], B, S, H, Hkv, hd)
    ry = oracle.out_proj(out, wo, bs[3], B, S, H, hd)
    rdout, rdwo, rdbo = oracle.out_proj_bwd(out, wo, dy, B, S, H, hd)
    rdx, rdws, rdbs = oracle.qkv_proj_bwd(x, *ws, gq, gk, gv, B, S, H, Hkv, hd)
    tol = TOL[dt]
    errs = {n: assert_close(n, host(g), ref, tol) for n, g, ref in (
        ("xq", xq, rq), ("xk", xk, rk), ("v", v, rv), ("y", y, ry), ("dout", dout, rdout),
        ("dwo", dwo, rdwo), ("dx", dx, rdx), ("dwq", dws[0], rdws[0]), ("dwk", dws[1], rdws[1]),
        ("dwv", dws[2], rdws[2]))}
    if bias:
        errs["dbo"] = assert_close("dbo", host(dbo), rdbo, tol)
        for n, g, ref in zip(("dbq", "dbk", "dbv"), dbs, rdbs):
            errs[n] = assert_close(n, host(g), ref, tol)
    print(shape, {k: f"{e:.2e}" for k, e in errs.items()})


@pytest.mark.parametrize("shape", [("bf16", 32, 1024, 12, 4, 64, 768, True),
                                   ("bf16", 1, 1024, 32, 8, 128, 4096, True)],
                         ids=["dim768_split_k", "qwen3_d4096"])
def test_projection_gradients_are_bitwise_reproducible(shape):
    """dx, the weight gradients (split over K and summed in split order where the output has
    few tiles) and the bias gradients are bitwise identical over repeated runs."""
    dt, B, S, H, Hkv, hd, d, bias = shape
    x, ws, wo, bs = _inputs(dt, B, S, H, Hkv, hd, d, bias, 650)
    note(f"projection determinism {shape}")
    pr = _proj(dt, B, S, H, Hkv, hd, ws, wo, bs)
    rng = np.random.default_rng(651)
    g = [dev(W.bf16_round(rng.standard_normal((B * n, S, hd), dtype=np.float32)), dt)
         for n in (H, Hkv, Hkv)]
    out, dy = g[0], dev(W.bf16_round(rng.standard_normal((B * S, d), dtype=np.float32)), dt)
    tx = dev(x, dt)
    runs = []
    for _ in range(3):
        dx, dws, dbs = pr.qkv_bwd(tx, *g)
        dout, dwo, dbo = pr.out_bwd(out, dy)
        torch.cuda.synchronize()
        runs.append([t.clone() for t in (dx, *dws, *dbs, dout, dwo, dbo)])
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_attention_block_matches_oracle_composition(dt):
    """x -> projections -> QK-norm + RoPE -> causal GQA attention -> output projection, forward
    and backward, against the oracle's composition of the same steps."""
    from causal_gqa_attention_amd.step import AttentionStep
    B, S, H, Hkv, hd, d = 2, 70, 4, 2, 64, 128
    x, ws, wo, bs = _inputs(dt, B, S, H, Hkv, hd, d, True, 640)
    rng = np.random.default_rng(641)
    gq_, gk_ = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32), \
        (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    dy = rng.standard_normal((B * S, d), dtype=np.float32)
    if dt == "bf16":
        dy = W.bf16_round(dy)
    eps, theta = 1e-5, 1e4
    note(f"attention block {dt}")
    pr = _proj(dt, B, S, H, Hkv, hd, ws, wo, bs)
    tx = dev(x, dt)
    xq, xk, v = pr.qkv_fwd(tx)
    step = AttentionStep(B, S, H, Hkv, hd, dt, eps, theta)
    step.xq.copy_(xq)
    step.xk.copy_(xk)
    step.v.copy_(v)
    step.gamma_q.copy_(torch.from_numpy(gq_))
    step.gamma_k.copy_(torch.from_numpy(gk_))
    step.forward()
    y = pr.out_fwd(step.out)
    dout, dwo, dbo = pr.out_bwd(step.out, dev(dy, dt))
    step.dout.copy_(dout)
    step.backward()
    dx, dws, dbs = pr.qkv_bwd(tx, step.dxq, step.dxk, step.dv)
    torch.cuda.synchronize()
    # oracle composition (float64 throughout, from the same rounded inputs)
    rq, rk, rv = oracle.qkv_proj(x, *ws, *bs[:3], B, S, H, Hkv, hd)
    f = oracle.forward(rq, rk, rv, gq_, gk_, H, Hkv, eps, theta)
    ry = oracle.out_proj(f["out"], wo, bs[3], B, S, H, hd)
    rdout, rdwo, _ = oracle.out_proj_bwd(f["out"], wo, dy, B, S, H, hd)
    g = oracle.backward(rq, rk, rv, gq_, gk_, rdout, H, Hkv, eps, theta)
    rdx, rdws, rdbs = oracle.qkv_proj_bwd(x, *ws, g["dxq"], g["dxk"], g["dv"], B, S, H, Hkv, hd)
    tol = TOL[dt]
    errs = {n: assert_close(n, host(a), ref, tol) for n, a, ref in (
        ("y", y, ry), ("dwo", dwo, rdwo), ("dx", dx, rdx), ("dwq", dws[0], rdws[0]),
        ("dwk", dws[1], rdws[1]), ("dwv", dws[2], rdws[2]), ("dbq", dbs[0], rdbs[0]),
        ("dgamma_q", step.dgamma_q, g["dgamma_q"]))}
    print(dt, {k: f"{e:.2e}" for k, e in errs.items()})
