"""Properties of the HIP path that hold exactly or at any size (GPU, through the C ABI):
GQA vs materialised repeat_kv, causal no-peeking, run-to-run determinism, constant V,
lse normalisation, single-token and zero-query closed forms."""
import math

import numpy as np
import pytest
import torch

import causal_gqa_attention_amd as X
import oracle
import workloads as W
from gpu_util import TOL, assert_close, dev, host, note, seeded_attention_inputs

pytestmark = pytest.mark.gpu


def _repeat_kv(t, H, Hkv):
    BKV, S, hd = t.shape
    B, group = BKV // Hkv, H // Hkv
    idx = [b * Hkv + qh // group for b in range(B) for qh in range(H)]
    return np.ascontiguousarray(t[idx])


@pytest.mark.parametrize("dtype,hd,S,H,Hkv", [
    ("bf16", 128, 300, 8, 2), ("bf16", 64, 257, 6, 3), ("f32", 64, 130, 4, 1),
    ("bf16", 128, 1000, 4, 1)])
def test_gqa_equals_mha_on_materialised_kv(dtype, hd, S, H, Hkv):
    """Per-query-head arithmetic does not depend on the group: out, lse and dq of GQA
    equal those of MHA on repeat_kv-materialised K/V bit for bit; dk/dv equal the group
    sum of the MHA per-head gradients within tolerance ("Phase T15: GQA", Decision 2)."""
    w = W.small_ragged(dtype, hd, S, 2, H, Hkv, index=300)
    q, k, v, do = seeded_attention_inputs(w, 77)
    note(f"gqa-vs-mha {dtype} hd{hd} S{S} H{H} kv{Hkv}")
    tq, tk, tv, td = (dev(a, dtype) for a in (q, k, v, do))
    out, lse = X.attn_fwd(tq, tk, tv, H, Hkv)
    dq, dk, dv = X.attn_bwd(tq, tk, tv, out, lse, td, H, Hkv)
    tk1, tv1 = dev(_repeat_kv(k, H, Hkv), dtype), dev(_repeat_kv(v, H, Hkv), dtype)
    out1, lse1 = X.attn_fwd(tq, tk1, tv1, H, H)
    dq1, dk1, dv1 = X.attn_bwd(tq, tk1, tv1, out1, lse1, td, H, H)
    torch.cuda.synchronize()
    assert torch.equal(out, out1) and torch.equal(lse, lse1) and torch.equal(dq, dq1)
    g = H // Hkv
    sk = host(dk1).reshape(-1, g, S, hd).sum(1)
    sv = host(dv1).reshape(-1, g, S, hd).sum(1)
    assert_close("dk group sum", host(dk), sk, TOL[dtype])
    assert_close("dv group sum", host(dv), sv, TOL[dtype])


@pytest.mark.parametrize("dtype,hd", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_causal_no_peeking_bitwise(dtype, hd):
    """Changing q, k, v after position t leaves out / lse at positions <= t bitwise
    unchanged; changing dout before t leaves dk / dv after t bitwise unchanged."""
    w = W.small_ragged(dtype, hd, 333, 1, 4, 2, index=301)
    q, k, v, do = seeded_attention_inputs(w, 5)
    t = 150
    q2, k2, v2, do2 = (a.copy() for a in (q, k, v, do))
    rng = np.random.default_rng(9)
    for a in (q2, k2, v2):
        a[:, t + 1:] = W.bf16_round(rng.standard_normal(a[:, t + 1:].shape, dtype=np.float32))
    do2[:, :t] = W.bf16_round(rng.standard_normal(do2[:, :t].shape, dtype=np.float32))
    note(f"causal invariance {dtype} hd{hd}")
    res = []
    for qq, kk, vv, dd in ((q, k, v, do), (q2, k2, v2, do), (q, k, v, do2)):
        tq, tk, tv, td = (dev(a, dtype) for a in (qq, kk, vv, dd))
        out, lse = X.attn_fwd(tq, tk, tv, 4, 2)
        dq, dk, dv = X.attn_bwd(tq, tk, tv, out, lse, td, 4, 2)
        torch.cuda.synchronize()
        res.append([host(a) for a in (out, lse.reshape(4, -1), dq, dk, dv)])
    a, b, c = res
    np.testing.assert_array_equal(b[0][:, :t + 1], a[0][:, :t + 1])
    np.testing.assert_array_equal(b[1][:, :t + 1], a[1][:, :t + 1])
    np.testing.assert_array_equal(c[3][:, t + 1:], a[3][:, t + 1:])
    np.testing.assert_array_equal(c[4][:, t + 1:], a[4][:, t + 1:])


# (workload, replaced fields): workloads 3 and 4 at full size run the shared-tile dk/dv
# kernel, workload 4 at batch 4 the private one, workload 5 the pipelined one, workload 2
# the generic fp32 kernels, workload 6 the generic bf16 kernels with the prologue backward
# in their dq / dk stores.
DETERMINISM = [(2, {}), (3, {}), (4, {}), (4, dict(batch=4)), (5, {}), (6, {})]


@pytest.mark.parametrize("idx,kw", DETERMINISM,
                         ids=[f"w{i}" + ("_" + "_".join(f"{k}{v}" for k, v in kw.items())
                                         if kw else "") for i, kw in DETERMINISM])
def test_backward_is_bitwise_reproducible(idx, kw):
    """out, lse, dq, dk, dv and dgamma are bitwise identical over repeated runs (no
    atomics; fixed reduction orders)."""
    from causal_gqa_attention_amd.step import AttentionStep
    w = W.WORKLOADS[idx].replace(**kw)
    x = W.make_inputs(w)
    note(f"determinism {w}")
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta).load(x.xq, x.xk, x.v, x.dout, x.gamma_q, x.gamma_k)
    outs = []
    for _ in range(5):
        step.run()
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (step.out, step.lse, step.dxq, step.dxk, step.dv,
                                          step.dgamma_q, step.dgamma_k)])
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_backward_reproducible_on_a_second_stream():
    """The same bits come out when the step runs on a non-default stream."""
    from causal_gqa_attention_amd.step import AttentionStep
    w = W.WORKLOADS[5].replace(seq_len=1024)
    x = W.make_inputs(w)
    step = AttentionStep(w.batch, w.seq_len, w.num_heads, w.num_kv_heads, w.head_dim, w.dtype,
                         w.eps, w.theta).load(x.xq, x.xk, x.v, x.dout, x.gamma_q, x.gamma_k)
    note("determinism across streams")
    step.run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.dxq, step.dxk, step.dv, step.dgamma_q)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        step.run(stream=s)
    s.synchronize()
    for a, b in zip(ref, (step.dxq, step.dxk, step.dv, step.dgamma_q)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_constant_v_and_lse_normalisation(dtype):
    w = W.small_ragged(dtype, 128, 400, 1, 4, 2, index=302)
    q, k, v, do = seeded_attention_inputs(w, 11)
    c = W.bf16_round(np.linspace(-2, 3, w.head_dim).astype(np.float32))
    vc = np.broadcast_to(c, v.shape).copy()
    note(f"constant v {dtype}")
    out, lse = X.attn_fwd(dev(q, dtype), dev(k, dtype), dev(vc, dtype), 4, 2)
    torch.cuda.synchronize()
    assert_close("out=const", host(out), np.broadcast_to(c, out.shape), TOL[dtype])
    # sum_j exp(s_ij - lse_i) = 1 with the float64 scores recomputed on the host
    lse = host(lse).reshape(w.bh, w.seq_len)
    for bh in range(w.bh):
        kv = bh // 2
        s = q[bh].astype(np.float64) @ k[kv].astype(np.float64).T / math.sqrt(w.head_dim)
        tot = np.array([np.exp(s[i, :i + 1] - lse[bh, i]).sum() for i in range(w.seq_len)])
        np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_queries_and_single_token_closed_forms(dtype):
    """q = 0: out_i = mean(v_0..v_i), lse_i = ln(i+1), dk = 0, dv_j = sum_{i>=j} dO_i/(i+1).
    S = 1: out = v, dq = dk = 0, dv = dO."""
    w = W.small_ragged(dtype, 64, 200, 1, 2, 1, index=303)
    q, k, v, do = seeded_attention_inputs(w, 12)
    q[...] = 0
    note(f"closed forms {dtype}")
    tq, tk, tv, td = (dev(a, dtype) for a in (q, k, v, do))
    out, lse = X.attn_fwd(tq, tk, tv, 2, 1)
    dq, dk, dv = X.attn_bwd(tq, tk, tv, out, lse, td, 2, 1)
    torch.cuda.synchronize()
    cnt = np.arange(1, w.seq_len + 1, dtype=np.float64)
    mean = np.cumsum(v[0].astype(np.float64), axis=0) / cnt[:, None]
    tol = TOL[dtype]
    for h in range(2):
        assert_close("out", host(out)[h], mean, tol)
    assert_close("lse", host(lse).reshape(2, -1), np.broadcast_to(np.log(cnt), (2, w.seq_len)), tol)
    assert np.abs(host(dk)).max() <= tol
    dsum = sum(do[h].astype(np.float64) / cnt[:, None] for h in range(2))
    assert_close("dv", host(dv)[0], np.cumsum(dsum[::-1], axis=0)[::-1], tol)
    # single token
    w1 = W.small_ragged(dtype, 64, 1, 3, 4, 2, index=304)
    q, k, v, do = seeded_attention_inputs(w1, 13)
    tq, tk, tv, td = (dev(a, dtype) for a in (q, k, v, do))
    out, lse = X.attn_fwd(tq, tk, tv, 4, 2)
    dq, dk, dv = X.attn_bwd(tq, tk, tv, out, lse, td, 4, 2)
    torch.cuda.synchronize()
    assert_close("out=v", host(out), _repeat_kv(v, 4, 2), tol)
    assert np.abs(host(dq)).max() <= 1e-4 and np.abs(host(dk)).max() <= 1e-4
    dvr = host(td).reshape(3, 2, 2, 1, 64).sum(2).reshape(6, 1, 64)
    assert_close("dv=sum dO", host(dv), dvr, tol)


def test_fused_prologue_backward_equals_separate_calls_f32():
    """fp32: xattn_bwd with the prologue equals xattn_bwd without it followed by
    xattn_qknorm_rope_bwd on Q and K, bit for bit."""
    w = W.WORKLOADS[2]
    x = W.make_inputs(w)
    note("fused vs separate prologue backward")
    cos, sin = X.rope_cache(w.seq_len, w.head_dim, w.theta)
    txq, txk, tv, td = (dev(a, "f32") for a in (x.xq, x.xk, x.v, x.dout))
    gq, gk = dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32")
    yq, rq = X.qknorm_rope_fwd(txq, gq, cos, sin, w.eps)
    yk, rk = X.qknorm_rope_fwd(txk, gk, cos, sin, w.eps)
    out, lse = X.attn_fwd(yq, yk, tv, w.num_heads, w.num_kv_heads)
    dxq, dxk, dv, dgq, dgk = X.attn_bwd(yq, yk, tv, out, lse, td, w.num_heads, w.num_kv_heads,
                                        prologue=dict(xq=txq, xk=txk, gamma_q=gq, gamma_k=gk,
                                                      rstd_q=rq, rstd_k=rk, cos_tab=cos,
                                                      sin_tab=sin))
    dyq, dyk, dv2 = X.attn_bwd(yq, yk, tv, out, lse, td, w.num_heads, w.num_kv_heads)
    dxq2, dgq2 = X.qknorm_rope_bwd(dyq, txq, gq, rq, cos, sin)
    dxk2, dgk2 = X.qknorm_rope_bwd(dyk, txk, gk, rk, cos, sin)
    torch.cuda.synchronize()
    for a, b in ((dxq, dxq2), (dxk, dxk2), (dv, dv2), (dgq, dgq2), (dgk, dgk2)):
        assert torch.equal(a, b)


# (workload, whether yq / rstd_q must equal the standalone prologue's bit for bit): the
# hd 64 / 128 bf16 forward sums the mean square in another order; the generic forward (bf16
# hd 16 / 32, fp32 every hd; key-split and unsplit kernels) repeats the standalone kernel's
# operations in its order.
QNORM_CASES = [
    (W.WORKLOADS[5].replace(seq_len=1000), False),
    (W.WORKLOADS[4].replace(batch=2, seq_len=300), False),
    (W.WORKLOADS[2], True),
    (W.WORKLOADS[6], True),
    (W.small_ragged("bf16", 16, 77, 2, 4, 2, index=305), True),
    (W.small_ragged("bf16", 16, 260, 8, 16, 4, index=306), True),
    (W.small_ragged("bf16", 32, 100, 1, 3, 1, index=307), True),
    (W.small_ragged("f32", 16, 77, 2, 4, 2, index=308), True),
    (W.small_ragged("f32", 32, 300, 4, 24, 6, index=309), True),
    (W.small_ragged("f32", 64, 300, 4, 24, 6, index=310), True),
    (W.small_ragged("f32", 128, 100, 1, 4, 2, theta=1e6, eps=1e-6, index=311), True),
]


@pytest.mark.parametrize("w,bitwise", QNORM_CASES,
                         ids=[f"{w.dtype}_hd{w.head_dim}_S{w.seq_len}_B{w.batch}"
                              for w, _ in QNORM_CASES])
def test_forward_with_fused_q_prologue_matches_separate_calls(w, bitwise):
    """xattn_fwd_qnorm: out and lse are bitwise those of xattn_fwd on the yq it wrote, and
    yq / rstd_q match xattn_qknorm_rope_fwd: bit for bit where the same operations run in
    the same order, else (bf16 at hd 64 / 128, whose in-kernel mean square sums in another
    order) rstd within a few ulp and yq within one rounding."""
    dtype = w.dtype
    x = W.make_inputs(w)
    note(f"fused Q prologue forward {w}")
    cos, sin = X.rope_cache(w.seq_len, w.head_dim, w.theta)
    txq, txk, tv = (dev(a, dtype) for a in (x.xq, x.xk, x.v))
    gq, gk = dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32")
    yk, _ = X.qknorm_rope_fwd(txk, gk, cos, sin, w.eps)
    out, lse, yq, rq = X.attn_fwd_qnorm(txq, gq, cos, sin, w.eps, yk, tv, w.num_heads,
                                        w.num_kv_heads)
    out2, lse2 = X.attn_fwd(yq, yk, tv, w.num_heads, w.num_kv_heads)
    yq2, rq2 = X.qknorm_rope_fwd(txq, gq, cos, sin, w.eps)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    if bitwise:
        assert torch.equal(yq, yq2) and torch.equal(rq, rq2)
    else:
        np.testing.assert_allclose(host(rq), host(rq2), rtol=2e-6, atol=0)
        d = (yq.float() - yq2.float()).abs()
        ulp = yq2.float().abs().clamp_min(2.0 ** -126) * 2.0 ** -7
        assert bool((d <= ulp).all()), float((d / ulp).max())


@pytest.mark.parametrize("dtype,hd,S,rows,docs", [
    ("f32", 16, 7, 3, None),        # one block, ragged position block
    ("f32", 128, 100, 8, None),
    ("bf16", 64, 77, 12, [30, 47]),  # positions restart per document
    ("bf16", 128, 300, 8, None),     # workload 5's K shape per position block
    ("bf16", 128, 33, 70, None),     # more rows than one pass: one position per block
    ("bf16", 32, 513, 5, [1, 500, 12])])
def test_prologue_with_table_equals_separate_calls(dtype, hd, S, rows, docs):
    """xattn_qknorm_rope_fwd_table: the table, y and rstd are bitwise those of
    xattn_rope_cache (or xattn_rope_cache_at) followed by xattn_qknorm_rope_fwd."""
    note(f"prologue with table {dtype} hd={hd} S={S} rows={rows} docs={docs}")
    rng = np.random.default_rng(hd * 1000 + S)
    x = dev(rng.standard_normal((rows, S, hd), dtype=np.float32), dtype)
    g = dev(1.0 + 0.1 * rng.standard_normal(hd).astype(np.float32), "f32")
    theta, eps = 1e4 if hd < 128 else 1e6, 1e-6
    pos = None if docs is None else X.segments(docs)[2]
    cos, sin = X.rope_cache(S, hd, theta) if pos is None else X.rope_cache_at(pos, hd, theta)
    y, r = X.qknorm_rope_fwd(x, g, cos, sin, eps)
    y2, r2, cos2, sin2 = X.qknorm_rope_fwd_table(x, g, theta, eps, positions=pos)
    torch.cuda.synchronize()
    for a, b in ((cos, cos2), (sin, sin2), (y, y2), (r, r2)):
        assert torch.equal(a, b)
