"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle on the same
seeded inputs.  Bar: norm-wise max relative error <= 1e-4 for fp32 io, <= 2e-2 for bf16
io, per output tensor.

Every comparison covers every element of every output: the small ragged shapes, and the
full-size workloads 3-5, whose whole step (every head, both dgamma) is compared with the
oracle run over the whole tensors.  Step outputs start as NaN, so an element that no
kernel writes fails.  Each comparison prints the norm-wise error and, as a diagnostic,
the elementwise p99 of |x - r| / (|r| + 1e-3 max|r|)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL, assert_close, attention_only, note, run_step, seeded_attention_inputs

pytestmark = pytest.mark.gpu

R = W.small_ragged
SMALL = [
    W.WORKLOADS[1],
    W.WORKLOADS[2],
    R("f32", 16, 7, 1, 2, 1, index=201),
    R("f32", 32, 77, 2, 6, 2, index=202),
    R("f32", 64, 130, 1, 4, 4, index=203),
    R("f32", 128, 100, 1, 4, 2, theta=1e6, eps=1e-6, index=204),
    R("f32", 64, 1, 2, 4, 2, index=205),
    R("bf16", 16, 33, 1, 3, 1, index=206),
    R("bf16", 32, 200, 2, 4, 4, index=207),
    R("bf16", 64, 77, 2, 6, 2, index=208),
    R("bf16", 64, 513, 1, 5, 1, index=209),
    R("bf16", 128, 257, 1, 8, 2, theta=1e6, eps=1e-6, index=210),
    R("bf16", 128, 1, 1, 4, 1, index=211),
    W.WORKLOADS[4].replace(batch=2, seq_len=190, index=212),
    W.WORKLOADS[5].replace(seq_len=300, index=213),
    # hd 128 shapes for the pipelined dk/dv kernel: MHA over two batch rows with a ragged
    # 64-key block; group 8 with the sequence exactly one 64-key block
    R("bf16", 128, 161, 2, 2, 2, theta=1e6, eps=1e-6, index=214),
    R("bf16", 128, 64, 1, 16, 2, index=215),
    # grids of >= 256 query workgroups: the generic forward / dq kernels without the key split
    # (the shapes above with fp32 or head_dim 16 / 32 run the split kernels)
    R("f32", 64, 300, 4, 24, 6, index=216),
    R("bf16", 16, 260, 8, 16, 4, index=217),
    # the generic dk/dv with the group's query heads split over workgroups (few key blocks):
    # group 5 over two splits, heads {0, 1} and {2, 3, 4}
    R("f32", 32, 1000, 2, 10, 2, index=218),
    # bf16 head_dim 16 / 32 apply the prologue backward in the dq / dk stores unless the
    # group is split as above: here with the dk/dv query walk split two ways (32 keys of 64
    # per wave); 207 and 217 cover the eight- and four-way splits, workload 6 the unsplit one
    R("bf16", 32, 520, 8, 32, 16, index=219),
    # a single token through both fused prologue halves of the generic bf16 kernels
    R("bf16", 16, 1, 3, 2, 2, index=220),
]
SMALL_IDS = [w.name if w.index < 100 else f"{w.dtype}_hd{w.head_dim}_S{w.seq_len}_"
             f"B{w.batch}_H{w.num_heads}_kv{w.num_kv_heads}" for w in SMALL]


def _compare_step(w, g, f, b):
    """Every output of the step against the oracle, every element."""
    tol = TOL[w.dtype]
    S = w.seq_len
    errs = {}
    for n in ("yq", "yk"):
        errs[n] = assert_close(n, g[n], f[n], tol)
    errs["rstd_q"] = assert_close("rstd_q", g["rstd_q"], f["rstd_q"].reshape(-1), tol)
    errs["rstd_k"] = assert_close("rstd_k", g["rstd_k"], f["rstd_k"].reshape(-1), tol)
    errs["out"] = assert_close("out", g["out"], f["out"], tol)
    errs["lse"] = assert_close("lse", g["lse"].reshape(-1, S), f["lse"], tol)
    for n in ("dxq", "dxk", "dv", "dgamma_q", "dgamma_k"):
        errs[n] = assert_close(n, g[n], b[n], tol)
    print(w.name, {k: f"{v:.2e}" for k, v in errs.items()})


@pytest.mark.parametrize("w", SMALL, ids=SMALL_IDS)
def test_step_matches_oracle(w):
    x = W.make_inputs(w)
    note(f"step {w}")
    g = run_step(w, x)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta)
    cos, sin = oracle.rope_tables(w.seq_len, w.head_dim, w.theta)
    np.testing.assert_allclose(g["cos"], cos, rtol=0, atol=2e-7)
    np.testing.assert_allclose(g["sin"], sin, rtol=0, atol=2e-7)
    _compare_step(w, g, f, b)


@pytest.mark.parametrize("w", SMALL, ids=SMALL_IDS)
def test_attention_matches_oracle(w):
    """Attention alone (q, k, v given directly): out, lse and dq, dk, dv."""
    q, k, v, do = seeded_attention_inputs(w, 1000 + w.index)
    note(f"attention {w}")
    g = attention_only(w, q, k, v, do)
    out, lse = oracle.attention_fwd(q, k, v, w.num_heads, w.num_kv_heads)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, w.num_heads, w.num_kv_heads)
    tol = TOL[w.dtype]
    errs = {n: assert_close(n, g[n], r, tol) for n, r in
            (("out", out), ("dq", dq), ("dk", dk), ("dv", dv))}
    errs["lse"] = assert_close("lse", g["lse"].reshape(lse.shape), lse, tol)
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


# Shapes whose dk/dv runs the shared-tile path (at least 1024 blocks of 128 keys); the
# second has 9 key tiles with a ragged last one.  Every head is compared.
SHARED_PATH = [
    W.small_ragged("bf16", 128, 200, 128, 8, 4, theta=1e4, eps=1e-5, index=230),
    W.small_ragged("bf16", 64, 1100, 16, 8, 8, theta=1e6, eps=1e-6, index=231),
]


@pytest.mark.parametrize("w", SHARED_PATH,
                         ids=[f"hd{w.head_dim}_S{w.seq_len}_B{w.batch}_H{w.num_heads}_kv{w.num_kv_heads}"
                              for w in SHARED_PATH])
def test_attention_shared_dkdv_path_matches_oracle(w):
    assert w.bkv * -(-w.seq_len // 128) >= 1024
    q, k, v, do = seeded_attention_inputs(w, 2000 + w.index)
    note(f"attention (shared dk/dv path) {w}")
    g = attention_only(w, q, k, v, do)
    out, lse = oracle.attention_fwd(q, k, v, w.num_heads, w.num_kv_heads)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, w.num_heads, w.num_kv_heads)
    tol = TOL[w.dtype]
    errs = {n: assert_close(n, x, r, tol) for n, x, r in
            (("out", g["out"], out), ("lse", g["lse"].reshape(lse.shape), lse),
             ("dq", g["dq"], dq), ("dk", g["dk"], dk), ("dv", g["dv"], dv))}
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


SHARED_PATH_STEP = [
    SHARED_PATH[0],
    W.small_ragged("bf16", 64, 100, 256, 8, 4, theta=1e4, eps=1e-6, index=232),
]


@pytest.mark.parametrize("w", SHARED_PATH_STEP,
                         ids=[f"hd{w.head_dim}_S{w.seq_len}_B{w.batch}" for w in SHARED_PATH_STEP])
def test_step_shared_dkdv_path_matches_oracle(w):
    """Whole step (prologue backward fused into the dk stores of the shared-tile dk/dv
    kernel), every head and dgamma compared."""
    assert w.bkv * -(-w.seq_len // 128) >= 1024
    x = W.make_inputs(w)
    note(f"step (shared dk/dv path) {w}")
    g = run_step(w, x)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta)
    _compare_step(w, g, f, b)


@pytest.mark.parametrize("idx", [3, 4, 5, 6])
def test_full_size_step_every_head(idx):
    """The workload at full size, in the configuration the benchmark times: every output of
    the step (prologue, attention forward, dq / dk / dv with the fused prologue backward,
    both dgamma) against the oracle over the whole tensors."""
    w = W.WORKLOADS[idx]
    x = W.make_inputs(w)
    note(f"full-size step {w}")
    g = run_step(w, x)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta)
    cos, sin = oracle.rope_tables(w.seq_len, w.head_dim, w.theta)
    np.testing.assert_allclose(g["cos"], cos, rtol=0, atol=2e-7)
    np.testing.assert_allclose(g["sin"], sin, rtol=0, atol=2e-7)
    _compare_step(w, g, f, b)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_prologue_matches_oracle_every_row(idx):
    """QK-norm + RoPE forward and backward on every row of the workload's Q and K, with
    the seeded dout (for Q) and v (for K) standing in for the upstream gradients."""
    import causal_gqa_attention_amd as X
    from gpu_util import dev, host
    w = W.WORKLOADS[idx]
    x = W.make_inputs(w)
    tol = TOL[w.dtype]
    note(f"prologue {w}")
    cos, sin = X.rope_cache(w.seq_len, w.head_dim, w.theta)
    for name, xin, gam, dy in (("q", x.xq, x.gamma_q, x.dout), ("k", x.xk, x.gamma_k, x.v)):
        tx, tg, tdy = dev(xin, w.dtype), dev(gam, "f32"), dev(dy, w.dtype)
        y, rstd = X.qknorm_rope_fwd(tx, tg, cos, sin, w.eps)
        dx, dg = X.qknorm_rope_bwd(tdy, tx, tg, rstd, cos, sin)
        ry, rr = oracle.qknorm_rope_fwd(xin, gam, w.eps, w.theta)
        rdx, rdg = oracle.qknorm_rope_bwd(dy, xin, gam, rr, w.theta)
        assert_close(f"y{name}", host(y), ry, tol)
        assert_close(f"rstd{name}", host(rstd), rr.reshape(-1), tol)
        assert_close(f"dx{name}", host(dx), rdx, tol)
        assert_close(f"dgamma{name}", host(dg), rdg, tol)


@pytest.mark.parametrize("wi,kw", [(5, dict(seq_len=300)), (4, dict(batch=2, seq_len=190)),
                                   (3, dict(batch=1, seq_len=257))])
def test_bf16_kernels_agree_with_the_fp32_kernels(wi, kw):
    """Cross-path gate (the pages' flash == composed check, here between two independent
    kernel sets): the bf16 kernels (bf16 io, fused prologue) and the generic fp32 kernels,
    run on the same bf16-valued inputs, agree within the bf16 band on every output."""
    w = W.WORKLOADS[wi].replace(**kw)
    x = W.make_inputs(w)  # bf16-valued inputs
    note(f"cross-path bf16 vs f32 {w}")
    gb = run_step(w, x)
    gf = run_step(w.replace(dtype="f32"), x)
    S = w.seq_len
    for n in ("yq", "yk", "rstd_q", "rstd_k", "out", "dxq", "dxk", "dv", "dgamma_q",
              "dgamma_k", "cos", "sin"):
        assert_close(n, gb[n], gf[n], TOL["bf16"])
    assert_close("lse", gb["lse"].reshape(-1, S), gf["lse"].reshape(-1, S), TOL["bf16"])
