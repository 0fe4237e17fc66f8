"""xattn_bwd_noalloc (the backward with the library's static scratch in place of a
workspace) against xattn_bwd (caller workspace) through the C ABI: two calls in a row, the
second on a smaller input, so the second runs on scratch that still holds the first call's
contents.  Both entry points run the same kernels, so the results must be bitwise equal;
they are also held to the oracle's bars (1e-4 fp32, 2e-2 bf16) on the small case."""
import numpy as np
import pytest
import torch

import causal_gqa_attention_amd as X
import oracle
import workloads as W
from causal_gqa_attention_amd.step import AttentionStep
from gpu_util import TOL, assert_close, host, note

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _forward(w):
    x = W.make_inputs(w)
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta).load(x.xq, x.xk, x.v, x.dout, x.gamma_q, x.gamma_k)
    step.forward()
    torch.cuda.synchronize()
    return x, step


def _outputs(step):
    f = lambda t: torch.full_like(t, NAN)
    pro = dict(step.prologue)
    pro["dgamma_q"], pro["dgamma_k"] = f(step.dgamma_q), f(step.dgamma_k)
    return f(step.yq), f(step.yk), f(step.v), pro


def _run(step, with_prologue, noalloc):
    dq, dk, dv, pro = _outputs(step)
    pro = pro if with_prologue else None
    args = (step.dims, step.yq, step.yk, step.v, step.out, step.lse, step.dout, dq, dk, dv, pro)
    if noalloc:
        X.xattn_bwd_noalloc(*args)
    else:
        X.xattn_bwd(*args, step.workspace)
    torch.cuda.synchronize()
    res = {"dq": dq, "dk": dk, "dv": dv}
    if pro is not None:
        res.update(dgamma_q=pro["dgamma_q"], dgamma_k=pro["dgamma_k"])
    return {n: t.clone() for n, t in res.items()}


# (larger, smaller) pairs: bf16 with the prologue fused into the gradient stores (hd 64,
# then hd 128; the generic kernels at hd 32, then hd 16), and the fp32 kernels with the
# separate prologue backward.
PAIRS = [
    (W.WORKLOADS[4].replace(batch=8, index=601), W.WORKLOADS[5].replace(seq_len=300, index=602)),
    (W.WORKLOADS[6].replace(batch=4, index=605), W.small_ragged("bf16", 16, 260, 8, 16, 4, index=606)),
    (W.WORKLOADS[2].replace(index=603), W.small_ragged("f32", 32, 77, 2, 6, 2, index=604)),
]


@pytest.mark.parametrize("big,small", PAIRS, ids=["bf16_fused_prologue", "bf16_generic_fused",
                                                  "f32"])
@pytest.mark.parametrize("with_prologue", [True, False], ids=["prologue", "attention_only"])
def test_noalloc_backward_matches_workspace_backward(big, small, with_prologue):
    (xb, sb), (xs, ss) = _forward(big), _forward(small)
    note(f"xattn_bwd_noalloc twice in a row: {big} then {small} prologue={with_prologue}")
    got = [_run(sb, with_prologue, True), _run(ss, with_prologue, True)]
    ref = [_run(sb, with_prologue, False), _run(ss, with_prologue, False)]
    for g, r in zip(got, ref):
        for n in r:
            assert torch.equal(g[n], r[n]), n
    if with_prologue:
        w, x = small, xs
        b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                            w.num_kv_heads, w.eps, w.theta)
        g = got[1]
        for n, r in (("dq", "dxq"), ("dk", "dxk"), ("dv", "dv"), ("dgamma_q", "dgamma_q"),
                     ("dgamma_k", "dgamma_k")):
            assert_close(n, host(g[n]), b[r], TOL[w.dtype])
