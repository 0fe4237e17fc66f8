"""CPU oracle for causal multi-head / grouped-query attention with a per-head
QK-RMSNorm + rotate_half RoPE prologue, forward and backward.

TEST INFRASTRUCTURE.  Only tests/, the package's smoke() check and the
benchmark's CPU-baseline leg may import or run this module; the HIP library and
its Python binding never do, and this module imports nothing from them.

Everything is computed in float64 with numpy.  Each function is the plain
definition written out, one (batch, head) at a time, with the full S x S score
matrix materialised; there is no tiling, no online softmax and no fusion.

Sources (titles of the pages and the section each function follows):
  * "Phase T9: Export to xserv", conventions table and Decision 1: RMSNorm
    x*rsqrt(mean(x^2)+eps)*gamma with no mean subtraction; QK-norm is a per-head
    RMSNorm over each [head_dim] vector, one gamma[head_dim] for all Q heads and
    one for all K heads, applied after the head reshape and before RoPE;
    rotate_half RoPE with frequency theta^(-2i/hd) and position = token index;
    scale 1/sqrt(head_dim); causal mask.
  * Mint documentation (morn.ink), section 5.3.1 (score, causal mask, stable
    softmax, weighted sum), 5.4.1-5.4.4 (rotation of pairs (i, i+hd/2), angle
    t*base^(-2i/dk), Q and K rotated but not V, backward = rotation by the
    negative angle, positions restart at 0 per sequence), 5.5.1-5.5.2 (RMSNorm
    forward and its backward: dot = sum g*dy*x, dx = g*dy/rms - x*dot/(d*rms^3),
    dg accumulated across rows).
  * "Phase T15: GQA", "what is GQA" and Decision 2: query head qh reads KV head
    qh // group with groups contiguous; the K/V gradient of a shared head is the
    sum over r < group of the gradients of query heads kvh*group + r.
  * "Phase T12: bf16 mixed precision", precision table: softmax, RoPE and norm in
    fp32 on the device; the oracle uses float64 throughout.
  * Mint documentation, section 10.3 (KV cache): a new token computes its own
    Q/K/V, appends K/V to the cache, and its query attends to every cached key;
    the result equals full-sequence attention (decode()).
  * Mint documentation, sections 5.3.1-5.3.2 (Q = X Wq + bq, K, V alike; output
    Concat(heads) Wo + bo, weights [d_in, d_out] applied as x @ W), "Phase T5: Tiny
    Transformer" layout pipeline (projection, reshape [seq, nh, hd], transpose to
    [nh, seq, hd] per head; merge back to [seq, nh*hd] before Wo) and "Phase T12"
    (linear GEMMs bf16 in / fp32 accumulate, gradients fp32): the projections below.
  * Mint documentation, section 8.2 (block-causal mask of a flattened batch:
    no attention across sample blocks, causal inside a block; RoPE positions
    numbered inside each sample): `segments` below, documents packed along the
    sequence axis, each a block of the mask with its own positions from 0.

Readings where the pages leave a step open (listed with the design notes):
  * masking: the pages use an additive -1e9 / -1e38 or a causal flag; all three
    exclude j > i exactly under a finite-input causal square attention, so the
    oracle excludes those entries exactly (they contribute exp(.) = 0);
  * lse (the forward's second output) is the natural-log logsumexp of the scaled,
    masked scores of each query row;
  * the attention backward is not written on the pages; it is the chain rule of
    the forward (dP = dO V^T, D = rowsum(P * dP), dS = P * (dP - D),
    dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd), dV = P^T dO), pinned by
    finite differences in the tests;
  * the group sum of K/V gradients runs over r in ascending order.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# RoPE (Mint docs 5.4.1 / 5.4.2; Phase T9 conventions table)
# --------------------------------------------------------------------------
def rope_tables(seq_len: int, head_dim: int, theta: float, pos_offset: int = 0):
    """cos/sin of the rotation angle t * theta^(-2i/hd), t = pos_offset + s for
    s in [0, seq_len), i in [0, hd/2).  Returns two [seq_len, hd/2] float64 arrays."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    t = np.arange(seq_len, dtype=np.float64) + pos_offset
    angle = t[:, None] * inv_freq[None, :]
    return np.cos(angle), np.sin(angle)


def rope_tables_at(positions, head_dim: int, theta: float):
    """cos/sin of the rotation angle p * theta^(-2i/hd) for explicit per-row positions p
    (the position of each token inside its own sample).  Returns two [len, hd/2] arrays."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / head_dim)
    angle = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(angle), np.sin(angle)


def segment_arrays(lengths):
    """Documents of the given lengths packed one after another along the sequence axis.
    Returns int64 arrays over the packed rows: lo (first row of the row's document), hi
    (its last row) and positions (row - lo: numbering restarts in every document)."""
    lengths = [int(n) for n in lengths]
    if any(n <= 0 for n in lengths):
        raise ValueError("document lengths must be positive")
    lo = np.concatenate([np.full(n, start) for n, start in
                         zip(lengths, np.cumsum([0] + lengths[:-1]))]).astype(np.int64)
    hi = np.concatenate([np.full(n, start + n - 1) for n, start in
                         zip(lengths, np.cumsum([0] + lengths[:-1]))]).astype(np.int64)
    return lo, hi, np.arange(len(lo), dtype=np.int64) - lo


def rope_apply(n, cos, sin):
    """rotate_half: pair (i, i + hd/2) rotated by the angle of (position, i).
    n: [..., S, hd]; cos/sin: [S, hd/2]."""
    n = _f64(n)
    half = n.shape[-1] // 2
    x, y = n[..., :half], n[..., half:]
    return np.concatenate([x * cos - y * sin, x * sin + y * cos], axis=-1)


def rope_apply_inverse(dy, cos, sin):
    """Rotation by the negative angle (the transpose of the rotation): this is the
    RoPE backward of Mint docs 5.4.4."""
    dy = _f64(dy)
    half = dy.shape[-1] // 2
    a, b = dy[..., :half], dy[..., half:]
    return np.concatenate([a * cos + b * sin, -a * sin + b * cos], axis=-1)


# --------------------------------------------------------------------------
# QK-norm = RMSNorm over each head vector (Mint docs 5.5.1, Phase T9 Decision 1)
# --------------------------------------------------------------------------
def qk_rmsnorm(x, gamma, eps: float):
    """n = x * gamma / rms with rms = sqrt(mean(x^2) + eps).  Returns (n, rstd)
    where rstd = 1/rms has the shape of x without its last axis."""
    x = _f64(x)
    gamma = _f64(gamma)
    d = x.shape[-1]
    ms = np.sum(x * x, axis=-1) / d
    rstd = 1.0 / np.sqrt(ms + eps)
    return x * rstd[..., None] * gamma, rstd


def qk_rmsnorm_bwd(dn, x, gamma, rstd):
    """Mint docs 5.5.2, per row: dot = sum_j g_j dy_j x_j;
    dx_j = g_j dy_j / rms - x_j dot / (d rms^3); dg_j = sum over rows of dy_j x_j / rms.
    Returns (dx, dgamma)."""
    dn, x, gamma, rstd = _f64(dn), _f64(x), _f64(gamma), _f64(rstd)
    d = x.shape[-1]
    r = rstd[..., None]
    dot = np.sum(gamma * dn * x, axis=-1, keepdims=True)
    dx = gamma * dn * r - x * dot * r ** 3 / d
    dgamma = np.sum((dn * x * r).reshape(-1, d), axis=0)
    return dx, dgamma


def _tables(S, hd, theta, pos_offset, positions):
    if positions is not None:
        return rope_tables_at(positions, hd, theta)
    return rope_tables(S, hd, theta, pos_offset)


def qknorm_rope_fwd(x, gamma, eps: float, theta: float, pos_offset: int = 0, positions=None):
    """Prologue forward on a [rows, S, hd] tensor: y = RoPE(QKnorm(x)); row s at position
    pos_offset + s, or positions[s] when given.  Returns (y, rstd[rows, S])."""
    x = _f64(x)
    _, S, hd = x.shape
    cos, sin = _tables(S, hd, theta, pos_offset, positions)
    n, rstd = qk_rmsnorm(x, gamma, eps)
    return rope_apply(n, cos, sin), rstd


def qknorm_rope_bwd(dy, x, gamma, rstd, theta: float, pos_offset: int = 0, positions=None):
    """Prologue backward: dn = RoPE^-1(dy), then the RMSNorm backward.
    Returns (dx, dgamma)."""
    x = _f64(x)
    _, S, hd = x.shape
    cos, sin = _tables(S, hd, theta, pos_offset, positions)
    dn = rope_apply_inverse(dy, cos, sin)
    return qk_rmsnorm_bwd(dn, x, gamma, rstd)


# --------------------------------------------------------------------------
# Causal GQA attention (Mint docs 5.3.1; Phase T15 head mapping)
# --------------------------------------------------------------------------
def _kv_index(bh: int, num_heads: int, num_kv_heads: int) -> int:
    b, qh = divmod(bh, num_heads)
    group = num_heads // num_kv_heads
    return b * num_kv_heads + qh // group


def _probs(qrow, krows, scale, seg_lo=None):
    """Scores s_ij = q_i.k_j * scale for j <= i (and j >= seg_lo[i], the first row of
    row i's document, when given), the rest excluded; returns (P, lse) with P the causal
    softmax (float64)."""
    S = qrow.shape[0]
    s = (qrow @ krows.T) * scale
    keep = np.tril(np.ones((S, S), dtype=bool))
    if seg_lo is not None:
        keep &= np.arange(S)[None, :] >= np.asarray(seg_lo)[:, None]
    s = np.where(keep, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.where(keep, np.exp(s - m), 0.0)
    l = np.sum(e, axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def _check_heads(num_heads, num_kv_heads):
    if num_kv_heads <= 0 or num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")


def attention_fwd(q, k, v, num_heads: int, num_kv_heads: int, heads=None, seg_lo=None):
    """q: [B*H, S, hd]; k, v: [B*Hkv, S, hd].  Returns (out [B*H,S,hd], lse [B*H,S]).
    `heads` optionally restricts the computation to a list of B*H row indices
    (the others stay zero).  seg_lo: optional [S] first row of each row's document
    (block-causal mask, the same packing for every batch row)."""
    _check_heads(num_heads, num_kv_heads)
    q, k, v = _f64(q), _f64(k), _f64(v)
    BH, S, hd = q.shape
    scale = 1.0 / np.sqrt(hd)
    out = np.zeros((BH, S, hd))
    lse = np.zeros((BH, S))
    for bh in (range(BH) if heads is None else heads):
        kv = _kv_index(bh, num_heads, num_kv_heads)
        p, lse[bh] = _probs(q[bh], k[kv], scale, seg_lo)
        out[bh] = p @ v[kv]
    return out, lse


def attention_bwd(q, k, v, dout, num_heads: int, num_kv_heads: int, kv_heads=None,
                  seg_lo=None):
    """Chain rule of attention_fwd.  Returns (dq, dk, dv) w.r.t. the q, k, v that
    attention_fwd consumed.  For each KV head the gradients of its `group` query
    heads are summed in ascending r.  `kv_heads` optionally restricts the work to a
    list of B*Hkv indices (and their query heads)."""
    _check_heads(num_heads, num_kv_heads)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    BH, S, hd = q.shape
    BKV = k.shape[0]
    group = num_heads // num_kv_heads
    scale = 1.0 / np.sqrt(hd)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for kv in (range(BKV) if kv_heads is None else kv_heads):
        b, kvh = divmod(kv, num_kv_heads)
        dk_sum = np.zeros((S, hd))
        dv_sum = np.zeros((S, hd))
        for r in range(group):
            bh = b * num_heads + kvh * group + r
            p, _ = _probs(q[bh], k[kv], scale, seg_lo)
            dp = dout[bh] @ v[kv].T                        # dP_ij = dO_i . v_j
            D = np.sum(p * dp, axis=1, keepdims=True)      # D_i = sum_j p_ij dP_ij
            ds = p * (dp - D)                              # dS_ij = p_ij (dP_ij - D_i)
            dq[bh] = (ds @ k[kv]) * scale
            dk_sum = dk_sum + (ds.T @ q[bh]) * scale
            dv_sum = dv_sum + p.T @ dout[bh]
        dk[kv] = dk_sum
        dv[kv] = dv_sum
    return dq, dk, dv


# --------------------------------------------------------------------------
# Whole path: prologue on Q and K, then attention
# --------------------------------------------------------------------------
def forward(xq, xk, v, gamma_q, gamma_k, num_heads, num_kv_heads, eps, theta,
            heads=None, pos_offset: int = 0, segments=None):
    """Returns a dict with yq, rstd_q, yk, rstd_k, out, lse.  segments: optional list of
    document lengths packed along the sequence axis (block-causal mask, positions
    restarting in every document)."""
    lo, pos = None, None
    if segments is not None:
        lo, _, pos = segment_arrays(segments)
    yq, rq = qknorm_rope_fwd(xq, gamma_q, eps, theta, pos_offset, pos)
    yk, rk = qknorm_rope_fwd(xk, gamma_k, eps, theta, pos_offset, pos)
    out, lse = attention_fwd(yq, yk, v, num_heads, num_kv_heads, heads, lo)
    return dict(yq=yq, rstd_q=rq, yk=yk, rstd_k=rk, out=out, lse=lse)


def backward(xq, xk, v, gamma_q, gamma_k, dout, num_heads, num_kv_heads, eps, theta,
             kv_heads=None, pos_offset: int = 0, segments=None):
    """Gradients of sum(dout * out) w.r.t. the raw inputs.  Returns a dict with
    dyq, dyk (w.r.t. the post-RoPE q, k), dxq, dxk, dv, dgamma_q, dgamma_k."""
    lo, pos = None, None
    if segments is not None:
        lo, _, pos = segment_arrays(segments)
    f = forward(xq, xk, v, gamma_q, gamma_k, num_heads, num_kv_heads, eps, theta,
                heads=[], pos_offset=pos_offset, segments=segments)
    dyq, dyk, dv = attention_bwd(f["yq"], f["yk"], v, dout, num_heads, num_kv_heads,
                                 kv_heads, lo)
    dxq, dgq = qknorm_rope_bwd(dyq, xq, gamma_q, f["rstd_q"], theta, pos_offset, pos)
    dxk, dgk = qknorm_rope_bwd(dyk, xk, gamma_k, f["rstd_k"], theta, pos_offset, pos)
    return dict(dyq=dyq, dyk=dyk, dxq=dxq, dxk=dxk, dv=dv, dgamma_q=dgq, dgamma_k=dgk)


# --------------------------------------------------------------------------
# KV-cache decode (Mint documentation 10.3)
# --------------------------------------------------------------------------
def decode(xq, xk, v, gamma_q, gamma_k, k_cache, v_cache, cache_len: int, num_heads: int,
           num_kv_heads: int, eps: float, theta: float):
    """One cached decode step.  The Sq new tokens of each sequence sit at positions
    cache_len .. cache_len + Sq - 1: their q, k get QK-norm + RoPE at those absolute
    positions, k and v are appended after the first cache_len rows of the caches, and
    new token i attends to the cached keys j <= cache_len + i of its KV head.
    xq: [B*H, Sq, hd]; xk, v: [B*Hkv, Sq, hd] (raw); k_cache, v_cache: [B*Hkv, >= cache_len,
    hd] (rotated keys and values of the earlier tokens; rows past cache_len are ignored).
    Returns (out [B*H, Sq, hd], lse [B*H, Sq], k_cache', v_cache' [B*Hkv, cache_len+Sq, hd])."""
    _check_heads(num_heads, num_kv_heads)
    yq, _ = qknorm_rope_fwd(xq, gamma_q, eps, theta, pos_offset=cache_len)
    yk, _ = qknorm_rope_fwd(xk, gamma_k, eps, theta, pos_offset=cache_len)
    kc = np.concatenate([_f64(k_cache)[:, :cache_len], yk], axis=1)
    vc = np.concatenate([_f64(v_cache)[:, :cache_len], _f64(v)], axis=1)
    BH, Sq, hd = yq.shape
    scale = 1.0 / np.sqrt(hd)
    out = np.zeros((BH, Sq, hd))
    lse = np.zeros((BH, Sq))
    for bh in range(BH):
        kv = _kv_index(bh, num_heads, num_kv_heads)
        for i in range(Sq):
            t = cache_len + i
            s = (kc[kv, :t + 1] @ yq[bh, i]) * scale  # every cached key at or before t
            m = s.max()
            e = np.exp(s - m)
            out[bh, i] = (e / e.sum()) @ vc[kv, :t + 1]
            lse[bh, i] = m + np.log(e.sum())
    return out, lse, kc, vc


# --------------------------------------------------------------------------
# Projections around attention (Mint documentation 5.3.1-5.3.2; Phase T5 layout pipeline)
# --------------------------------------------------------------------------
def split_heads(m, batch: int, seq_len: int, heads: int, head_dim: int):
    """[B*S, heads*hd] (token rows, head-major columns) -> [B*heads, S, hd]: the reshape to
    [seq, nh, hd] and the transpose that makes each head's [seq, hd] block contiguous."""
    m = _f64(m)
    return np.ascontiguousarray(m.reshape(batch, seq_len, heads, head_dim)
                                .transpose(0, 2, 1, 3).reshape(batch * heads, seq_len, head_dim))


def merge_heads(t, batch: int, seq_len: int, heads: int, head_dim: int):
    """Inverse of split_heads: [B*heads, S, hd] -> [B*S, heads*hd]."""
    t = _f64(t)
    return np.ascontiguousarray(t.reshape(batch, heads, seq_len, head_dim)
                                .transpose(0, 2, 1, 3).reshape(batch * seq_len, heads * head_dim))


def _affine(x, w, b):
    y = _f64(x) @ _f64(w)
    return y if b is None else y + _f64(b)[None, :]


def qkv_proj(x, wq, wk, wv, bq, bk, bv, batch, seq_len, num_heads, num_kv_heads, head_dim):
    """x: [B*S, d] token rows; wq: [d, H*hd], wk, wv: [d, Hkv*hd]; biases None or [out].
    Returns (xq [B*H, S, hd], xk, v [B*Hkv, S, hd]): q = x Wq + bq split into heads, etc."""
    return (split_heads(_affine(x, wq, bq), batch, seq_len, num_heads, head_dim),
            split_heads(_affine(x, wk, bk), batch, seq_len, num_kv_heads, head_dim),
            split_heads(_affine(x, wv, bv), batch, seq_len, num_kv_heads, head_dim))


def out_proj(out, wo, bo, batch, seq_len, num_heads, head_dim):
    """out: [B*H, S, hd]; wo: [H*hd, d]; bo None or [d].  y = merge_heads(out) Wo + bo,
    [B*S, d]."""
    return _affine(merge_heads(out, batch, seq_len, num_heads, head_dim), wo, bo)


def out_proj_bwd(out, wo, dy, batch, seq_len, num_heads, head_dim):
    """Chain rule of out_proj.  Returns (dout [B*H, S, hd], dwo [H*hd, d], dbo [d])."""
    dy = _f64(dy)
    om = merge_heads(out, batch, seq_len, num_heads, head_dim)
    dout = split_heads(dy @ _f64(wo).T, batch, seq_len, num_heads, head_dim)
    return dout, om.T @ dy, dy.sum(axis=0)


def qkv_proj_bwd(x, wq, wk, wv, dxq, dxk, dv, batch, seq_len, num_heads, num_kv_heads,
                 head_dim):
    """Chain rule of qkv_proj.  Returns dx [B*S, d] and (dwq, dwk, dwv), (dbq, dbk, dbv)."""
    x = _f64(x)
    dq = merge_heads(dxq, batch, seq_len, num_heads, head_dim)
    dk = merge_heads(dxk, batch, seq_len, num_kv_heads, head_dim)
    dvm = merge_heads(dv, batch, seq_len, num_kv_heads, head_dim)
    dx = dq @ _f64(wq).T + dk @ _f64(wk).T + dvm @ _f64(wv).T
    return dx, (x.T @ dq, x.T @ dk, x.T @ dvm), (dq.sum(axis=0), dk.sum(axis=0), dvm.sum(axis=0))
