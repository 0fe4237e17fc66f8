"""Parity of the block-causal mask over packed documents (Mint documentation 8.2: a flattened
batch masked block by block, RoPE positions counted inside each sample) with the float64
oracle: the whole step (prologue with per-document positions, attention forward and
backward, fused prologue backward, dgamma) against oracle.forward / oracle.backward with the
same document lengths, under the usual norm-wise bars (1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from causal_gqa_attention_amd.step import AttentionStep
from gpu_util import TOL, assert_close, note, poison

pytestmark = pytest.mark.gpu

R = W.small_ragged
CASES = [
    # bf16 hd 128, private dk/dv kernel; a one-token document and boundaries inside tiles
    (R("bf16", 128, 300, 1, 8, 2, theta=1e6, eps=1e-6, index=501), [100, 1, 37, 162]),
    # bf16 hd 64, documents on 64-row stage boundaries and one spanning several tiles
    (R("bf16", 64, 257, 2, 6, 2, index=502), [64, 64, 129]),
    # bf16 hd 128 and hd 64 on the shared-tile dk/dv kernel (>= 1024 workgroups of 128 keys)
    (R("bf16", 128, 200, 128, 8, 4, index=503), [50, 50, 100]),
    (R("bf16", 64, 200, 128, 8, 4, index=504), [3, 97, 100]),
    # generic kernels: fp32 hd 64 and hd 16 (every document a single token), bf16 hd 32
    (R("f32", 64, 150, 2, 4, 2, index=505), [10, 70, 1, 69]),
    (R("f32", 16, 40, 1, 2, 1, index=506), [1] * 40),
    (R("bf16", 32, 77, 1, 4, 2, index=507), [30, 47]),
    # bf16 head_dim 16 / 32 with the prologue backward in the dq / dk stores (no group
    # split): MHA, and GQA group 2 on the unsplit dq kernel
    (R("bf16", 32, 150, 2, 4, 4, index=513), [1, 60, 89]),
    (R("bf16", 16, 90, 2, 4, 4, index=514), [45, 2, 43]),
    (R("bf16", 32, 300, 12, 8, 4, index=515), [128, 100, 72]),
]
IDS = [f"{w.dtype}_hd{w.head_dim}_S{w.seq_len}_B{w.batch}_docs{len(d)}" for w, d in CASES]


def _step(w, x, docs):
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta, doc_lengths=docs)
    step.load(x.xq, x.xk, x.v, x.dout, x.gamma_q, x.gamma_k)
    poison(step)
    step.run()
    torch.cuda.synchronize()
    return step.results()


@pytest.mark.parametrize("w,docs", CASES, ids=IDS)
def test_step_with_documents_matches_oracle(w, docs):
    x = W.make_inputs(w)
    note(f"documents {docs[:6]}... {w}")
    g = _step(w, x, docs)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta, segments=docs)
    b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta, segments=docs)
    _, _, pos = oracle.segment_arrays(docs)
    cos, sin = oracle.rope_tables_at(pos, w.head_dim, w.theta)
    np.testing.assert_allclose(g["cos"], cos, rtol=0, atol=2e-7)
    np.testing.assert_allclose(g["sin"], sin, rtol=0, atol=2e-7)
    tol = TOL[w.dtype]
    errs = {n: assert_close(n, g[n], f[n], tol) for n in ("yq", "yk", "out")}
    errs["lse"] = assert_close("lse", g["lse"].reshape(f["lse"].shape), f["lse"], tol)
    for n in ("dxq", "dxk", "dv", "dgamma_q", "dgamma_k"):
        errs[n] = assert_close(n, g[n], b[n], tol)
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


def test_documents_full_size_qwen_shape_every_head():
    """The long-context shape at full size packed as four documents: every output of the
    step against the oracle over the whole tensors."""
    w = W.WORKLOADS[5]
    docs = [1000, 37, 2048, 1011]
    x = W.make_inputs(w)
    note(f"documents {docs} full size {w}")
    g = _step(w, x, docs)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta, segments=docs)
    b = oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta, segments=docs)
    tol = TOL[w.dtype]
    errs = {n: assert_close(n, g[n], f[n], tol) for n in ("yq", "yk", "out")}
    errs["lse"] = assert_close("lse", g["lse"].reshape(f["lse"].shape), f["lse"], tol)
    for n in ("dxq", "dxk", "dv", "dgamma_q", "dgamma_k"):
        errs[n] = assert_close(n, g[n], b[n], tol)
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


def test_document_masking_is_bitwise_reproducible():
    w = R("bf16", 128, 520, 1, 8, 2, theta=1e6, eps=1e-6, index=508)
    docs = [200, 5, 315]
    x = W.make_inputs(w)
    note(f"documents determinism {w}")
    a, b = _step(w, x, docs), _step(w, x, docs)
    for n in ("out", "lse", "dxq", "dxk", "dv", "dgamma_q", "dgamma_k"):
        np.testing.assert_array_equal(a[n], b[n])


# One document spanning the whole sequence sees exactly the plain causal mask, but runs the
# document code: every stage that holds the diagonal or the ragged end goes through the
# per-element range test, where without documents the diagonal stages only mask each wave's
# diagonal sub-tile in place.  The two must give the same bits.
WHOLE = [
    R("bf16", 128, 300, 1, 8, 2, theta=1e6, eps=1e-6, index=509),  # pipelined dk/dv, hd 128
    R("bf16", 128, 200, 128, 8, 4, index=510),                     # shared dk/dv, hd 128
    R("bf16", 64, 330, 96, 6, 6, index=511),                       # shared dk/dv, hd 64
    R("bf16", 64, 1000, 4, 12, 4, index=512),                      # private dk/dv, hd 64
]


@pytest.mark.parametrize("w", WHOLE, ids=[f"hd{w.head_dim}_S{w.seq_len}_B{w.batch}"
                                          for w in WHOLE])
def test_one_whole_document_equals_no_documents(w):
    x = W.make_inputs(w)
    note(f"whole-sequence document against none {w}")
    a, b = _step(w, x, [w.seq_len]), _step(w, x, None)
    for n in ("yq", "yk", "out", "lse", "dxq", "dxk", "dv", "dgamma_q", "dgamma_k"):
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
