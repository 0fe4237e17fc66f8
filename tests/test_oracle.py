"""Pins for the CPU oracle: closed forms, invariants, library special cases,
brute force and finite differences, each tied to what the pages fix.

No test here touches the GPU or the HIP library.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import oracle.brute as brute
import oracle.oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY_GQA = W.Workload(90, "tiny_gqa", 1, 8, 6, 2, 8, "f32", "perturbed", 1e-5, 1e4)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _inputs(w, seed=None):
    return W.make_inputs(w, seed)


def _fwd(w, x, **kw):
    return oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads,
                          w.num_kv_heads, w.eps, w.theta, **kw)


def _bwd(w, x, **kw):
    return oracle.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                           w.num_kv_heads, w.eps, w.theta, **kw)


def _repeat_kv(t, H, Hkv):
    """Materialise K/V heads as "Phase T15: GQA" Decision 1 states it:
    out[b*H + qh] = in[b*Hkv + qh // group]."""
    BKV, S, hd = t.shape
    B = BKV // Hkv
    group = H // Hkv
    out = np.empty((B * H, S, hd), dtype=t.dtype)
    for b in range(B):
        for qh in range(H):
            out[b * H + qh] = t[b * Hkv + qh // group]
    return out


def _scores(q, k):
    return (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) / math.sqrt(q.shape[-1])


# ---------------------------------------------------------------------------
# brute force vs vectorised
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("w", [W.WORKLOADS[1], TINY_GQA], ids=["cfg1", "tiny_gqa"])
def test_brute_force_matches_vectorised(w):
    x = _inputs(w)
    f, fb = _fwd(w, x), brute.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k,
                                      w.num_heads, w.num_kv_heads, w.eps, w.theta)
    for key in ("yq", "yk", "rstd_q", "rstd_k", "out", "lse"):
        np.testing.assert_allclose(f[key], np.array(fb[key]), rtol=0, atol=1e-12, err_msg=key)
    b = _bwd(w, x)
    bb = brute.backward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, x.dout, w.num_heads,
                        w.num_kv_heads, w.eps, w.theta)
    for key in b:
        np.testing.assert_allclose(b[key], np.array(bb[key]), rtol=0, atol=1e-12, err_msg=key)


def test_brute_force_matches_vectorised_gqa_f32_workload_slice():
    # workload 2's head shape (8 heads / 2 KV heads, hd 64) on a short sequence
    w = W.WORKLOADS[2].replace(batch=1, seq_len=6)
    x = _inputs(w)
    f = _fwd(w, x)
    fb = brute.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads,
                       w.num_kv_heads, w.eps, w.theta)
    np.testing.assert_allclose(f["out"], np.array(fb["out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(f["lse"], np.array(fb["lse"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# softmax / output closed forms (Mint docs 5.3.1 steps 2-5)
# ---------------------------------------------------------------------------
def test_softmax_rows_sum_to_one_and_lse_normalises():
    w = TINY_GQA.replace(seq_len=33)
    x = _inputs(w)
    f = _fwd(w, x)
    S = w.seq_len
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        p, lse = O._probs(f["yq"][bh], f["yk"][kv], 1 / math.sqrt(w.head_dim))
        np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
        assert np.all(np.triu(p, 1) == 0.0)
        s = _scores(f["yq"][bh], f["yk"][kv])
        tot = np.array([np.exp(s[i, :i + 1] - f["lse"][bh, i]).sum() for i in range(S)])
        np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


def test_lse_matches_library_logsumexp():
    w = TINY_GQA.replace(seq_len=21)
    x = _inputs(w)
    f = _fwd(w, x)
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        s = _scores(f["yq"][bh], f["yk"][kv])
        ref = np.array([scipy.special.logsumexp(s[i, :i + 1]) for i in range(w.seq_len)])
        np.testing.assert_allclose(f["lse"][bh], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("mask_value", [float(r[0]) for r in _read_golden("mask_constants.txt")])
def test_exact_exclusion_equals_additive_mask(mask_value):
    """The pages add -1e9 (Phase T5) or -1e38 (Mint 5.3.1) above the diagonal
    before a plain softmax; the oracle excludes those entries exactly."""
    w = TINY_GQA.replace(seq_len=19)
    x = _inputs(w)
    f = _fwd(w, x)
    S = w.seq_len
    mask = np.triu(np.full((S, S), mask_value), 1)
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        p = scipy.special.softmax(_scores(f["yq"][bh], f["yk"][kv]) + mask, axis=1)
        np.testing.assert_allclose(f["out"][bh], p @ x.v[kv].astype(np.float64), rtol=0, atol=1e-13)


def test_constant_v_returns_the_constant():
    w = TINY_GQA.replace(seq_len=40)
    x = _inputs(w)
    c = np.linspace(-2, 3, w.head_dim)
    v = np.broadcast_to(c, x.v.shape).copy()
    out, _ = oracle.attention_fwd(x.xq, x.xk, v, w.num_heads, w.num_kv_heads)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=0, atol=1e-14)


def test_row_zero_reads_only_itself():
    w = TINY_GQA.replace(seq_len=12)
    x = _inputs(w)
    f = _fwd(w, x)
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        np.testing.assert_array_equal(f["out"][bh, 0], x.v[kv, 0].astype(np.float64))
        s00 = f["yq"][bh, 0] @ f["yk"][kv, 0] / math.sqrt(w.head_dim)
        assert abs(f["lse"][bh, 0] - s00) <= 1e-14 * max(1.0, abs(s00))


def test_zero_queries_closed_form():
    """xq = 0 gives y_q = 0 (the prologue maps 0 to 0) and all scores 0: then
    out_i = mean(v_0..v_i), lse_i = ln(i+1), dv_j = sum_{i>=j} dO_i/(i+1), dk = 0."""
    w = TINY_GQA.replace(seq_len=13)
    x = _inputs(w)
    x.xq[...] = 0.0
    f = _fwd(w, x)
    b = _bwd(w, x)
    S = w.seq_len
    assert np.all(f["yq"] == 0.0)
    cnt = np.arange(1, S + 1, dtype=np.float64)
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        mean = np.cumsum(x.v[kv].astype(np.float64), axis=0) / cnt[:, None]
        np.testing.assert_allclose(f["out"][bh], mean, rtol=0, atol=1e-14)
        np.testing.assert_allclose(f["lse"][bh], np.log(cnt), rtol=0, atol=1e-14)
    np.testing.assert_array_equal(b["dyk"], 0.0)
    for kv in range(w.bkv):
        bb, kvh = divmod(kv, w.num_kv_heads)
        heads = [bb * w.num_heads + kvh * w.group + r for r in range(w.group)]
        do = sum(x.dout[h].astype(np.float64) / cnt[:, None] for h in heads)
        ref = np.cumsum(do[::-1], axis=0)[::-1]
        np.testing.assert_allclose(b["dv"][kv], ref, rtol=0, atol=1e-13)


def test_single_token_closed_form():
    w = TINY_GQA.replace(seq_len=1)
    x = _inputs(w)
    f = _fwd(w, x)
    b = _bwd(w, x)
    np.testing.assert_allclose(f["out"], _repeat_kv(x.v, w.num_heads, w.num_kv_heads),
                               rtol=0, atol=0)
    np.testing.assert_array_equal(b["dyq"], 0.0)
    np.testing.assert_array_equal(b["dyk"], 0.0)
    dv = np.zeros_like(b["dv"])
    for bh in range(w.bh):
        dv[O._kv_index(bh, w.num_heads, w.num_kv_heads)] += x.dout[bh]
    np.testing.assert_allclose(b["dv"], dv, rtol=0, atol=1e-15)


def test_score_bound():
    """RoPE preserves norms (Mint 5.4.3) and the normalised row has RMS <= max|gamma|,
    so |s_ij| <= max|gamma_q| max|gamma_k| sqrt(hd)."""
    w = TINY_GQA.replace(seq_len=30)
    x = _inputs(w)
    x.xq *= 50.0
    f = _fwd(w, x)
    bound = np.abs(x.gamma_q).max() * np.abs(x.gamma_k).max() * math.sqrt(w.head_dim)
    for bh in range(w.bh):
        kv = O._kv_index(bh, w.num_heads, w.num_kv_heads)
        assert np.abs(_scores(f["yq"][bh], f["yk"][kv])).max() <= bound * (1 + 1e-12)


# ---------------------------------------------------------------------------
# GQA mapping and the repeat_kv group sum ("Phase T15: GQA")
# ---------------------------------------------------------------------------
def test_golden_head_map():
    rows = _read_golden("gqa_head_map_h8_kv2.txt")
    H, Hkv, S, hd = 8, 2, 5, 4
    rng = np.random.default_rng(0)
    q = rng.standard_normal((H, S, hd))
    k = rng.standard_normal((Hkv, S, hd))
    # KV head h carries the constant value h: the output then names the KV head read
    v = np.stack([np.full((S, hd), float(h)) for h in range(Hkv)])
    out, _ = oracle.attention_fwd(q, k, v, H, Hkv)
    for qh, kvh in rows:
        np.testing.assert_allclose(out[int(qh)], float(kvh), rtol=0, atol=1e-14)


@pytest.mark.parametrize("H,Hkv", [(6, 2), (6, 3), (4, 1), (6, 6)])
def test_gqa_equals_mha_on_materialised_kv_bitwise(H, Hkv):
    w = TINY_GQA.replace(batch=2, num_heads=H, num_kv_heads=Hkv, seq_len=11)
    x = _inputs(w)
    f = _fwd(w, x)
    kk = _repeat_kv(f["yk"], H, Hkv)
    vv = _repeat_kv(x.v.astype(np.float64), H, Hkv)
    out, lse = oracle.attention_fwd(f["yq"], kk, vv, H, H)
    np.testing.assert_array_equal(out, f["out"])
    np.testing.assert_array_equal(lse, f["lse"])


@pytest.mark.parametrize("H,Hkv", [(6, 2), (6, 3), (4, 1)])
def test_repeat_kv_backward_is_the_group_sum(H, Hkv):
    w = TINY_GQA.replace(batch=2, num_heads=H, num_kv_heads=Hkv, seq_len=9)
    x = _inputs(w)
    f = _fwd(w, x)
    dq, dk, dv = oracle.attention_bwd(f["yq"], f["yk"], x.v, x.dout, H, Hkv)
    kk = _repeat_kv(f["yk"], H, Hkv)
    vv = _repeat_kv(x.v.astype(np.float64), H, Hkv)
    dq1, dk1, dv1 = oracle.attention_bwd(f["yq"], kk, vv, x.dout, H, H)
    np.testing.assert_array_equal(dq, dq1)
    group = H // Hkv
    for kv in range(w.bkv):
        b, kvh = divmod(kv, Hkv)
        rows = [b * H + kvh * group + r for r in range(group)]
        sk = np.zeros_like(dk[kv])
        sv = np.zeros_like(dv[kv])
        for r in rows:          # ascending r, as "Phase T15: GQA" Decision 2 sums
            sk = sk + dk1[r]
            sv = sv + dv1[r]
        np.testing.assert_allclose(dk[kv], sk, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dv[kv], sv, rtol=0, atol=1e-13)


def test_mqa_is_the_single_kv_head_case():
    H, S, hd = 5, 10, 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((H, S, hd))
    k = rng.standard_normal((1, S, hd))
    v = rng.standard_normal((1, S, hd))
    out, lse = oracle.attention_fwd(q, k, v, H, 1)
    for h in range(H):
        o1, l1 = oracle.attention_fwd(q[h:h + 1], k, v, 1, 1)
        np.testing.assert_array_equal(out[h], o1[0])
        np.testing.assert_array_equal(lse[h], l1[0])


def test_library_sdpa_cross_check():
    """torch CPU float64 scaled_dot_product_attention(is_causal=True) on
    repeat_interleave(group)-expanded K/V ("Phase T15: GQA", PyTorch parity),
    forward and autograd backward."""
    w = TINY_GQA.replace(batch=2, seq_len=17, num_heads=6, num_kv_heads=2, head_dim=8)
    x = _inputs(w)
    f = _fwd(w, x)
    b = _bwd(w, x)
    B, H, Hkv, S, hd = w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim
    q = torch.tensor(f["yq"].reshape(B, H, S, hd), requires_grad=True)
    k = torch.tensor(f["yk"].reshape(B, Hkv, S, hd), requires_grad=True)
    v = torch.tensor(x.v.astype(np.float64).reshape(B, Hkv, S, hd), requires_grad=True)
    kk = k.repeat_interleave(w.group, dim=1)
    vv = v.repeat_interleave(w.group, dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True)
    out.backward(torch.tensor(x.dout.astype(np.float64).reshape(B, H, S, hd)))
    np.testing.assert_allclose(out.detach().numpy().reshape(B * H, S, hd), f["out"], atol=1e-13)
    np.testing.assert_allclose(q.grad.numpy().reshape(B * H, S, hd), b["dyq"], atol=1e-12)
    np.testing.assert_allclose(k.grad.numpy().reshape(B * Hkv, S, hd), b["dyk"], atol=1e-12)
    np.testing.assert_allclose(v.grad.numpy().reshape(B * Hkv, S, hd), b["dv"], atol=1e-12)


# ---------------------------------------------------------------------------
# causality: no peeking at the future (Mint docs 5.3.1 step 3)
# ---------------------------------------------------------------------------
def test_future_perturbation_leaves_past_bitwise():
    w = TINY_GQA.replace(seq_len=24)
    x = _inputs(w)
    f = _fwd(w, x)
    b = _bwd(w, x)
    t = 10
    y = _inputs(w)
    rng = np.random.default_rng(7)
    for a in (y.xq, y.xk, y.v):
        a[:, t + 1:] = rng.standard_normal(a[:, t + 1:].shape).astype(np.float32)
    g = _fwd(w, y)
    np.testing.assert_array_equal(g["out"][:, :t + 1], f["out"][:, :t + 1])
    np.testing.assert_array_equal(g["lse"][:, :t + 1], f["lse"][:, :t + 1])
    # perturbing dO at rows < t leaves dk_j, dv_j for j > t bitwise unchanged
    z = _inputs(w)
    z.dout[:, :t] = rng.standard_normal(z.dout[:, :t].shape).astype(np.float32)
    bz = _bwd(w, z)
    np.testing.assert_array_equal(bz["dyk"][:, t + 1:], b["dyk"][:, t + 1:])
    np.testing.assert_array_equal(bz["dv"][:, t + 1:], b["dv"][:, t + 1:])


# ---------------------------------------------------------------------------
# RoPE (Mint docs 5.4.1-5.4.4; Phase T9 conventions)
# ---------------------------------------------------------------------------
def test_rope_hd2_is_complex_multiplication_by_exp_it():
    """With hd = 2 the only pair has frequency theta^0 = 1, so position t rotates by
    t radians: (y0 + i y1) = (x0 + i x1) * exp(i t)."""
    S = 50
    rng = np.random.default_rng(1)
    n = rng.standard_normal((3, S, 2))
    cos, sin = oracle.rope_tables(S, 2, 1e4)
    y = oracle.rope_apply(n, cos, sin)
    z = (n[..., 0] + 1j * n[..., 1]) * np.exp(1j * np.arange(S))
    np.testing.assert_allclose(y[..., 0], z.real, atol=1e-12)
    np.testing.assert_allclose(y[..., 1], z.imag, atol=1e-12)


@pytest.mark.parametrize("hd,theta", [(16, 1e4), (64, 1e4), (128, 1e6)])
def test_rope_frequency_ladder(hd, theta):
    """Per pair i the angle at position 1 is theta^(-2i/hd): the first is 1, and
    the ladder is geometric with ratio theta^(-2/hd) (Mint 5.4.2)."""
    cos, sin = oracle.rope_tables(2, hd, theta)
    ang = np.arctan2(sin[1], cos[1])
    assert ang[0] == 1.0
    ratios = ang[1:] / ang[:-1]
    np.testing.assert_allclose(ratios, theta ** (-2.0 / hd), rtol=1e-12)
    # one step past the last pair the ladder reaches 1/theta exactly
    np.testing.assert_allclose(ang[-1] * theta ** (-2.0 / hd), 1.0 / theta, rtol=1e-12)


def test_rope_frequency_ends_golden():
    rows = {r[0]: (float(r[1]), float(r[2])) for r in _read_golden("rope_frequency_ends.txt")}
    hd = 128
    cos, sin = oracle.rope_tables(2, hd, 1e4)
    ang = np.arctan2(sin[1], cos[1])
    f0, tol0 = rows["first"]
    assert ang[0] == f0
    fl, toll = rows["last"]
    assert abs(ang[-1] - fl) <= toll * fl


def test_rope_position_zero_identity_norm_and_inverse():
    rng = np.random.default_rng(2)
    S, hd = 64, 32
    n = rng.standard_normal((4, S, hd))
    cos, sin = oracle.rope_tables(S, hd, 1e4)
    y = oracle.rope_apply(n, cos, sin)
    np.testing.assert_array_equal(y[:, 0], n[:, 0])
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(n, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.rope_apply_inverse(y, cos, sin), n, atol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    """Mint 5.4.3: q_t^R . k_j^R depends on positions only through t - j."""
    rng = np.random.default_rng(4)
    S, hd = 20, 16
    q = rng.standard_normal((1, S, hd))
    k = rng.standard_normal((1, S, hd))
    for theta in (1e4, 1e6):
        c0, s0 = oracle.rope_tables(S, hd, theta, 0)
        c1, s1 = oracle.rope_tables(S, hd, theta, 37)
        a = oracle.rope_apply(q, c0, s0)[0] @ oracle.rope_apply(k, c0, s0)[0].T
        b = oracle.rope_apply(q, c1, s1)[0] @ oracle.rope_apply(k, c1, s1)[0].T
        np.testing.assert_allclose(a, b, atol=1e-11)


def test_rope_only_rotates_q_and_k():
    """V is not rotated (Mint 5.4.4): shifting the positions of q and k together
    (the same content at pos_offset c) leaves the attention output unchanged."""
    w = TINY_GQA.replace(seq_len=15)
    x = _inputs(w)
    f0 = _fwd(w, x)
    f1 = _fwd(w, x, pos_offset=11)
    np.testing.assert_allclose(f1["out"], f0["out"], atol=1e-12)


# ---------------------------------------------------------------------------
# QK-norm = RMSNorm (Mint docs 5.5; Phase T9 Decision 1)
# ---------------------------------------------------------------------------
def test_qknorm_matches_library_rms_norm_and_its_autograd():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 9, 16)) * 3
    g = 1 + 0.1 * rng.standard_normal(16)
    dn = rng.standard_normal(x.shape)
    eps = 1e-5
    n, rstd = O.qk_rmsnorm(x, g, eps)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    nt = torch.nn.functional.rms_norm(xt, (16,), gt, eps)
    np.testing.assert_allclose(n, nt.detach().numpy(), atol=1e-13)
    nt.backward(torch.tensor(dn))
    dx, dg = O.qk_rmsnorm_bwd(dn, x, g, rstd)
    np.testing.assert_allclose(dx, xt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), atol=1e-12)


def test_qknorm_unit_gamma_is_not_identity_and_has_unit_rms():
    """Phase T9 Decision 1: with gamma = 1 QK-norm still rescales each head vector
    to RMS sqrt(ms / (ms + eps))."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 7, 64)) * 5
    eps = 1e-5
    n, _ = oracle.qk_rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)
    assert np.abs(n - x).max() > 1.0


# ---------------------------------------------------------------------------
# gradients: central finite differences in float64 (the pages' L = sum(W * out) harness)
# ---------------------------------------------------------------------------
def _fd_check(w, x, h=1e-6, tol=1e-6, segments=None):
    def loss(xq, xk, v, gq, gk):
        out = oracle.forward(xq, xk, v, gq, gk, w.num_heads, w.num_kv_heads, w.eps,
                             w.theta, segments=segments)["out"]
        return float(np.sum(out * x.dout))

    base = [np.asarray(a, np.float64).copy() for a in (x.xq, x.xk, x.v, x.gamma_q, x.gamma_k)]
    g = oracle.backward(*base, x.dout, w.num_heads, w.num_kv_heads, w.eps, w.theta,
                        segments=segments)
    names = ["dxq", "dxk", "dv", "dgamma_q", "dgamma_k"]
    for idx, name in enumerate(names):
        arr = base[idx]
        num = np.zeros(arr.size)
        flat = arr.reshape(-1)
        for e in range(arr.size):
            old = flat[e]
            flat[e] = old + h
            lp = loss(*base)
            flat[e] = old - h
            lm = loss(*base)
            flat[e] = old
            num[e] = (lp - lm) / (2 * h)
        ana = np.asarray(g[name]).reshape(-1)
        err = np.abs(num - ana).max() / max(np.abs(ana).max(), 1e-30)
        assert err < tol, (name, err)


@pytest.mark.parametrize("w", [W.WORKLOADS[1], TINY_GQA], ids=["cfg1", "tiny_gqa_h6_kv2_hd8"])
def test_finite_difference_gradcheck(w):
    _fd_check(w, _inputs(w))


def test_finite_difference_gradcheck_attention_only():
    """dq, dk, dv of attention alone (w.r.t. the post-RoPE q, k and v)."""
    w = TINY_GQA.replace(seq_len=6)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((w.bh, w.seq_len, w.head_dim))
    k = rng.standard_normal((w.bkv, w.seq_len, w.head_dim))
    v = rng.standard_normal((w.bkv, w.seq_len, w.head_dim))
    do = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, w.num_heads, w.num_kv_heads)
    h = 1e-6
    for arr, ana in ((q, dq), (k, dk), (v, dv)):
        flat = arr.reshape(-1)
        num = np.zeros(arr.size)
        for e in range(arr.size):
            old = flat[e]
            flat[e] = old + h
            lp = np.sum(oracle.attention_fwd(q, k, v, w.num_heads, w.num_kv_heads)[0] * do)
            flat[e] = old - h
            lm = np.sum(oracle.attention_fwd(q, k, v, w.num_heads, w.num_kv_heads)[0] * do)
            flat[e] = old
            num[e] = (lp - lm) / (2 * h)
        err = np.abs(num - ana.reshape(-1)).max() / np.abs(ana).max()
        assert err < 1e-6


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------
def test_planted_head_map_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(O, "_kv_index", lambda bh, H, Hkv: (bh // H) * Hkv + (bh % H) % Hkv)
    with pytest.raises(AssertionError):
        test_golden_head_map()


def test_planted_rope_backward_sign_mistake_is_caught(monkeypatch):
    def bad(dy, cos, sin):
        dy = np.asarray(dy, np.float64)
        half = dy.shape[-1] // 2
        a, b = dy[..., :half], dy[..., half:]
        return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)
    monkeypatch.setattr(O, "rope_apply_inverse", bad)
    with pytest.raises(AssertionError):
        _fd_check(TINY_GQA, _inputs(TINY_GQA))


def test_planted_missing_eps_is_caught(monkeypatch):
    real = O.qk_rmsnorm
    monkeypatch.setattr(O, "qk_rmsnorm", lambda x, g, eps: real(x, g, 0.0))
    with pytest.raises(AssertionError):
        test_qknorm_matches_library_rms_norm_and_its_autograd()


def test_planted_transposed_dk_mistake_is_caught(monkeypatch):
    real_bwd = O.attention_bwd

    def bad(q, k, v, dout, H, Hkv, kv_heads=None, seg_lo=None):
        dq, dk, dv = real_bwd(q, k, v, dout, H, Hkv, kv_heads, seg_lo)
        return dq, dk[:, ::-1].copy(), dv
    monkeypatch.setattr(O, "attention_bwd", bad)
    with pytest.raises(AssertionError):
        _fd_check(TINY_GQA, _inputs(TINY_GQA))


# --------------------------------------------------------------------------
# KV-cache decode (Mint documentation 10.3: cached decoding equals full-sequence
# attention; the pages' own check is token-by-token cached inference against one
# full-sequence pass)
# --------------------------------------------------------------------------
def _decode_all(x, w, q_len):
    """Run O.decode over the whole sequence in steps of q_len new tokens from an empty
    cache; returns the stacked (out, lse) and the final caches."""
    S = w.seq_len
    kc = np.zeros((w.bkv, 0, w.head_dim))
    vc = np.zeros((w.bkv, 0, w.head_dim))
    outs, lses = [], []
    for t in range(0, S, q_len):
        n = min(q_len, S - t)
        o, l, kc, vc = O.decode(x.xq[:, t:t + n], x.xk[:, t:t + n], x.v[:, t:t + n],
                                x.gamma_q, x.gamma_k, kc, vc, t, w.num_heads,
                                w.num_kv_heads, w.eps, w.theta)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1), kc, vc


@pytest.mark.parametrize("q_len", [1, 3])
def test_cached_decode_equals_full_sequence(q_len):
    w = W.small_ragged("f32", 32, 17, 2, 6, 2, theta=1e4, eps=1e-5, index=301)
    x = W.make_inputs(w)
    f = O.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads, w.eps,
                  w.theta)
    out, lse, kc, vc = _decode_all(x, w, q_len)
    np.testing.assert_allclose(out, f["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, f["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(kc, f["yk"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(vc, x.v.astype(np.float64))


def test_decode_step_matches_library_sdpa_on_the_cache():
    """One new token at position t: softmax(q k^T / sqrt(hd)) v over cache rows 0..t, by
    torch's float64 scaled_dot_product_attention (no mask: every cached key is visible)."""
    w = W.small_ragged("f32", 16, 9, 1, 4, 2, index=302)
    x = W.make_inputs(w)
    t = 8
    yk, _ = O.qknorm_rope_fwd(x.xk[:, :t], x.gamma_k, w.eps, w.theta)
    out, lse, kc, vc = O.decode(x.xq[:, t:], x.xk[:, t:], x.v[:, t:], x.gamma_q, x.gamma_k, yk,
                                x.v[:, :t], t, w.num_heads, w.num_kv_heads, w.eps, w.theta)
    yq, _ = O.qknorm_rope_fwd(x.xq[:, t:], x.gamma_q, w.eps, w.theta, pos_offset=t)
    group = w.num_heads // w.num_kv_heads
    q = torch.from_numpy(yq)                                   # [H, 1, hd]
    k = torch.from_numpy(kc).repeat_interleave(group, dim=0)   # [H, t+1, hd]
    v = torch.from_numpy(vc).repeat_interleave(group, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    s = (q @ k.transpose(1, 2)).numpy()[:, 0] / math.sqrt(w.head_dim)
    np.testing.assert_allclose(lse[:, 0], scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_planted_decode_position_mistake_is_caught(monkeypatch):
    """New tokens rotated as if they sat at position 0 (the absolute position dropped):
    cached decoding no longer equals the full sequence."""
    w = W.small_ragged("f32", 16, 6, 1, 2, 1, index=303)
    x = W.make_inputs(w)
    f = O.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads, w.eps,
                  w.theta)
    real = O.qknorm_rope_fwd
    monkeypatch.setattr(O, "qknorm_rope_fwd",
                        lambda xx, g, eps, theta, pos_offset=0: real(xx, g, eps, theta, 0))
    out, _, _, _ = _decode_all(x, w, 1)
    assert np.abs(out - f["out"]).max() > 1e-3


# --------------------------------------------------------------------------
# Block-causal mask over packed documents (Mint documentation 8.2: a flattened batch
# is masked block by block, no attention across samples, causal inside; RoPE positions
# counted inside each sample)
# --------------------------------------------------------------------------
def _pack(a, B, heads):
    """[B*heads, S, hd] -> [heads, B*S, hd]: the batch's samples one after another."""
    _, S, hd = a.shape
    return np.ascontiguousarray(a.reshape(B, heads, S, hd).transpose(1, 0, 2, 3)
                                .reshape(heads, B * S, hd))


def _unpack(a, B, heads):
    """Inverse of _pack for [heads, B*S, ...] arrays."""
    S = a.shape[1] // B
    rest = a.shape[2:]
    return np.ascontiguousarray(a.reshape((heads, B, S) + rest).transpose((1, 0, 2) + tuple(
        range(3, 3 + len(rest)))).reshape((B * heads, S) + rest))


def test_segment_arrays():
    lo, hi, pos = O.segment_arrays([3, 1, 2])
    np.testing.assert_array_equal(lo, [0, 0, 0, 3, 4, 4])
    np.testing.assert_array_equal(hi, [2, 2, 2, 3, 5, 5])
    np.testing.assert_array_equal(pos, [0, 1, 2, 0, 0, 1])
    with pytest.raises(ValueError):
        O.segment_arrays([2, 0])


def test_block_causal_flattened_batch_equals_batched():
    """The pages' case: a batch of B samples of length S flattened to one row of B*S with
    blocks of S gives, sample by sample, exactly the batched causal attention (forward,
    backward, prologue with positions restarting per sample)."""
    w = W.small_ragged("f32", 16, 7, 3, 4, 2, index=310)
    x = _inputs(w)
    B, H, Hkv = w.batch, w.num_heads, w.num_kv_heads
    f = _fwd(w, x)
    g = _bwd(w, x)
    fx = oracle.forward(_pack(x.xq, B, H), _pack(x.xk, B, Hkv), _pack(x.v, B, Hkv), x.gamma_q,
                        x.gamma_k, H, Hkv, w.eps, w.theta, segments=[w.seq_len] * B)
    gx = oracle.backward(_pack(x.xq, B, H), _pack(x.xk, B, Hkv), _pack(x.v, B, Hkv), x.gamma_q,
                         x.gamma_k, _pack(x.dout, B, H), H, Hkv, w.eps, w.theta,
                         segments=[w.seq_len] * B)
    for name, heads in (("out", H), ("lse", H), ("yq", H), ("yk", Hkv)):
        np.testing.assert_allclose(_unpack(fx[name], B, heads), f[name], rtol=0, atol=1e-12)
    for name, heads in (("dxq", H), ("dxk", Hkv), ("dv", Hkv)):
        np.testing.assert_allclose(_unpack(gx[name], B, heads), g[name], rtol=0, atol=1e-12)
    for name in ("dgamma_q", "dgamma_k"):
        np.testing.assert_allclose(gx[name], g[name], rtol=1e-12, atol=1e-12)


def test_single_segment_is_plain_causal():
    w = W.small_ragged("f32", 32, 11, 1, 4, 1, index=311)
    x = _inputs(w)
    a, b = _fwd(w, x), _fwd(w, x, segments=[w.seq_len])
    for n in ("out", "lse", "yq", "yk"):
        np.testing.assert_array_equal(a[n], b[n])


def test_segmented_attention_scalar_definition():
    """Row i of a document starting at lo_i: softmax over keys lo_i <= j <= i only, written
    out with scalar loops."""
    rng = np.random.default_rng(312)
    S, hd, segs = 9, 4, [2, 4, 1, 2]
    q, k, v = (rng.standard_normal((1, S, hd)) for _ in range(3))
    lo, _, _ = O.segment_arrays(segs)
    out, lse = O.attention_fwd(q, k, v, 1, 1, seg_lo=lo)
    for i in range(S):
        keys = range(int(lo[i]), i + 1)
        s = [sum(q[0, i, d] * k[0, j, d] for d in range(hd)) / math.sqrt(hd) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        for d in range(hd):
            ref = sum(e[n] * v[0, j, d] for n, j in enumerate(keys)) / z
            assert abs(out[0, i, d] - ref) < 1e-12
        assert abs(lse[0, i] - (m + math.log(z))) < 1e-12


def test_segmented_finite_difference_gradcheck():
    _fd_check(TINY_GQA, _inputs(TINY_GQA), segments=[3, 1, 4])


def test_planted_missing_segment_mask_is_caught(monkeypatch):
    """A mask that forgets the document boundary (plain causal) breaks the flattened-batch
    equality."""
    real = O._probs
    monkeypatch.setattr(O, "_probs", lambda q, k, scale, seg_lo=None: real(q, k, scale))
    with pytest.raises(AssertionError):
        test_block_causal_flattened_batch_equals_batched()


# --------------------------------------------------------------------------
# Projections (Mint documentation 5.3.1-5.3.2; Phase T5 layout pipeline)
# --------------------------------------------------------------------------
def _proj_inputs(seed, B=2, S=3, H=4, Hkv=2, hd=4, d=6, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B * S, d))
    wq = rng.standard_normal((d, H * hd))
    wk = rng.standard_normal((d, Hkv * hd))
    wv = rng.standard_normal((d, Hkv * hd))
    wo = rng.standard_normal((H * hd, d))
    bs = [rng.standard_normal(n) if bias else None for n in (H * hd, Hkv * hd, Hkv * hd, d)]
    return x, wq, wk, wv, wo, bs


def test_projection_scalar_definition_and_head_layout():
    """q_t = x_t Wq + bq (row vector times matrix), then head h of token (b, s) is columns
    h*hd .. h*hd + hd - 1 of that row, at [b*H + h, s]; written out with scalar loops."""
    B, S, H, Hkv, hd, d = 2, 3, 4, 2, 4, 6
    x, wq, wk, wv, wo, (bq, bk, bv, bo) = _proj_inputs(320)
    xq, xk, v = O.qkv_proj(x, wq, wk, wv, bq, bk, bv, B, S, H, Hkv, hd)
    for b in range(B):
        for s in range(S):
            for h in range(H):
                for e in range(hd):
                    c = h * hd + e
                    ref = sum(x[b * S + s, i] * wq[i, c] for i in range(d)) + bq[c]
                    assert abs(xq[b * H + h, s, e] - ref) < 1e-12
            for h in range(Hkv):
                for e in range(hd):
                    c = h * hd + e
                    ref = sum(x[b * S + s, i] * wv[i, c] for i in range(d)) + bv[c]
                    assert abs(v[b * Hkv + h, s, e] - ref) < 1e-12
    out = np.random.default_rng(321).standard_normal((B * H, S, hd))
    y = O.out_proj(out, wo, bo, B, S, H, hd)
    for b in range(B):
        for s in range(S):
            for j in range(d):
                ref = sum(out[b * H + h, s, e] * wo[h * hd + e, j]
                          for h in range(H) for e in range(hd)) + bo[j]
                assert abs(y[b * S + s, j] - ref) < 1e-12
    np.testing.assert_array_equal(O.merge_heads(O.split_heads(x @ wq, B, S, H, hd), B, S, H, hd),
                                  x @ wq)


def test_projection_backward_finite_differences():
    B, S, H, Hkv, hd, d = 1, 3, 2, 1, 4, 5
    x, wq, wk, wv, wo, (bq, bk, bv, bo) = _proj_inputs(322, B, S, H, Hkv, hd, d)
    rng = np.random.default_rng(323)
    gq = rng.standard_normal((B * H, S, hd))
    gk = rng.standard_normal((B * Hkv, S, hd))
    gv = rng.standard_normal((B * Hkv, S, hd))
    dy = rng.standard_normal((B * S, d))
    out = rng.standard_normal((B * H, S, hd))

    def loss_in(x_, wq_, wk_, wv_, bq_, bk_, bv_):
        q, k, v = O.qkv_proj(x_, wq_, wk_, wv_, bq_, bk_, bv_, B, S, H, Hkv, hd)
        return float(np.sum(q * gq) + np.sum(k * gk) + np.sum(v * gv))

    def loss_out(out_, wo_, bo_):
        return float(np.sum(O.out_proj(out_, wo_, bo_, B, S, H, hd) * dy))

    dx, (dwq, dwk, dwv), (dbq, dbk, dbv) = O.qkv_proj_bwd(x, wq, wk, wv, gq, gk, gv, B, S, H,
                                                          Hkv, hd)
    dout, dwo, dbo = O.out_proj_bwd(out, wo, dy, B, S, H, hd)

    def fd(f, args, i):
        a = args[i]
        g = np.zeros(a.size)
        for e in range(a.size):
            old = a.flat[e]
            a.flat[e] = old + 1e-6
            up = f(*args)
            a.flat[e] = old - 1e-6
            dn = f(*args)
            a.flat[e] = old
            g[e] = (up - dn) / 2e-6
        return g.reshape(a.shape)

    ins = [x, wq, wk, wv, bq, bk, bv]
    for i, ref in enumerate([dx, dwq, dwk, dwv, dbq, dbk, dbv]):
        np.testing.assert_allclose(fd(loss_in, ins, i), ref, rtol=1e-6, atol=1e-6)
    outs = [out, wo, bo]
    for i, ref in enumerate([dout, dwo, dbo]):
        np.testing.assert_allclose(fd(loss_out, outs, i), ref, rtol=1e-6, atol=1e-6)


def test_projection_without_bias_is_plain_product():
    x, wq, wk, wv, wo, _ = _proj_inputs(324, bias=False)
    q, _, _ = O.qkv_proj(x, wq, wk, wv, None, None, None, 2, 3, 4, 2, 4)
    np.testing.assert_array_equal(O.merge_heads(q, 2, 3, 4, 4), x @ wq)
