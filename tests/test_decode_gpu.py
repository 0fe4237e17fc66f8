"""Parity of the KV-cache decode (xattn_decode) with the float64 oracle.

The pages' own check (Mint documentation 10.3) is that token-by-token cached inference
equals one full-sequence pass; here the GPU decodes a whole sequence in steps of q_len new
tokens into its own caches and is compared with the oracle's full-sequence forward (out,
lse, and the appended rotated keys / values), under the same norm-wise bars as the rest
of the path (1e-4 for fp32 io, 2e-2 for bf16).  Full-size shapes prefill the cache with
the library's prologue and decode the last tokens, compared on every head."""
import numpy as np
import pytest
import torch

import causal_gqa_attention_amd as X
import oracle
import workloads as W
from gpu_util import TOL, TDT, assert_close, dev, host, note

pytestmark = pytest.mark.gpu

R = W.small_ragged
# (workload, q_len, spare cache rows past the sequence)
STEPWISE = [
    (W.WORKLOADS[1], 1, 0),                                            # tiny MHA, fp32
    (R("f32", 64, 40, 2, 8, 2, index=401), 1, 5),                      # GQA g4
    (R("f32", 128, 33, 1, 4, 1, theta=1e6, eps=1e-6, index=402), 3, 2),  # MQA, 3 at a time
    (R("f32", 32, 21, 1, 16, 2, index=403), 2, 0),                     # g8, R = 16
    (R("bf16", 128, 70, 1, 8, 2, theta=1e6, eps=1e-6, index=404), 1, 1),  # Qwen-like g4
    (R("bf16", 64, 50, 2, 6, 2, index=405), 2, 3),                     # g3, R = 6
    (R("bf16", 32, 20, 1, 4, 4, index=406), 5, 0),                     # MHA, 5 at a time
    (R("bf16", 16, 9, 1, 2, 1, index=407), 4, 1),                      # hd 16, ragged last
    # rows per KV head against what one wave holds (16 for fp32 and for bf16 at hd 64 / 128,
    # 8 for bf16 at hd 16 / 32): beyond it, row chunks
    (R("bf16", 128, 70, 1, 32, 8, theta=1e6, eps=1e-6, index=409), 4, 2),  # Qwen3 heads, R 16
    (R("f32", 64, 40, 1, 16, 2, index=410), 4, 0),                     # g8, R = 32
    (R("bf16", 64, 50, 1, 8, 1, index=411), 3, 1),                     # MQA g8, R = 24, ragged
    (R("bf16", 128, 48, 1, 4, 1, index=412), 16, 0),                   # R = 64, 4 chunks
]
IDS = [f"{w.dtype}_hd{w.head_dim}_S{w.seq_len}_H{w.num_heads}_kv{w.num_kv_heads}_q{q}"
       for w, q, _ in STEPWISE]


def _decode_sequence(w, x, q_len, spare):
    """Decode the whole sequence on the GPU in steps of q_len from an empty cache."""
    S, cap = w.seq_len, w.seq_len + spare
    dt = w.dtype
    cos, sin = X.rope_cache(cap, w.head_dim, w.theta)
    txq, txk, tv = dev(x.xq, dt), dev(x.xk, dt), dev(x.v, dt)
    gq, gk = dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32")
    kc = torch.zeros((w.bkv, cap, w.head_dim), dtype=TDT[dt], device="cuda")
    vc = torch.zeros_like(kc)
    dims = X.make_decode_dims(txq[:, :q_len], kc, w.num_heads, w.num_kv_heads, cap - q_len)
    ws = torch.empty(X.xattn_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    outs, lses = [], []
    for t in range(0, S, q_len):
        n = min(q_len, S - t)
        sl = slice(t, t + n)
        o, l = X.decode(txq[:, sl].contiguous(), txk[:, sl].contiguous(), tv[:, sl].contiguous(),
                        gq, gk, cos, sin, w.eps, kc, vc, t, w.num_heads, w.num_kv_heads,
                        workspace=ws)
        outs.append(o)
        lses.append(l.reshape(-1, n))
    torch.cuda.synchronize()
    return (host(torch.cat(outs, dim=1)), host(torch.cat(lses, dim=1)), host(kc), host(vc))


@pytest.mark.parametrize("w,q_len,spare", STEPWISE, ids=IDS)
def test_cached_decode_matches_full_sequence(w, q_len, spare):
    x = W.make_inputs(w)
    note(f"decode stepwise q_len={q_len} {w}")
    out, lse, kc, vc = _decode_sequence(w, x, q_len, spare)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    tol = TOL[w.dtype]
    errs = {"out": assert_close("out", out, f["out"], tol),
            "lse": assert_close("lse", lse, f["lse"], tol),
            "k_cache": assert_close("k_cache", kc[:, :w.seq_len], f["yk"], tol)}
    np.testing.assert_array_equal(vc[:, :w.seq_len], x.v.astype(np.float64))
    assert not kc[:, w.seq_len:].any() and not vc[:, w.seq_len:].any()  # rows past: untouched
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


def test_decode_is_bitwise_reproducible():
    w = R("bf16", 128, 300, 2, 8, 2, theta=1e6, eps=1e-6, index=408)
    x = W.make_inputs(w)
    note(f"decode determinism {w}")
    a = _decode_sequence(w, x, 2, 0)
    b = _decode_sequence(w, x, 2, 0)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# Full-size shapes: the cache holds S - q_len tokens (prefilled with the library's prologue
# on the same raw keys), then one decode step; every head compared.
FULL = [(W.WORKLOADS[5].replace(batch=2), 1), (W.WORKLOADS[4], 2), (W.WORKLOADS[2], 4)]


@pytest.mark.parametrize("w,q_len", FULL, ids=[f"{w.name}_q{q}" for w, q in FULL])
def test_full_size_decode_last_tokens(w, q_len):
    x = W.make_inputs(w)
    S, dt = w.seq_len, w.dtype
    pos = S - q_len
    note(f"decode full size {w} pos={pos} q_len={q_len}")
    cos, sin = X.rope_cache(S, w.head_dim, w.theta)
    txk, tv = dev(x.xk, dt), dev(x.v, dt)
    gq, gk = dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32")
    yk, _ = X.qknorm_rope_fwd(txk[:, :pos].contiguous(), gk, cos, sin, w.eps)
    kc = torch.zeros((w.bkv, S, w.head_dim), dtype=TDT[dt], device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :pos] = yk
    vc[:, :pos] = tv[:, :pos]
    xq_new = dev(x.xq[:, pos:], dt)
    dims = X.make_decode_dims(xq_new, kc, w.num_heads, w.num_kv_heads, pos)
    out = torch.full_like(xq_new, float("nan"))
    lse = torch.full((xq_new.shape[0] * q_len,), float("nan"), dtype=torch.float32,
                     device="cuda")
    ws = torch.empty(X.xattn_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    X.xattn_decode(dims, xq_new, txk[:, pos:].contiguous(), tv[:, pos:].contiguous(), gq, gk,
                   cos, sin, w.eps, kc, vc, out, lse, ws)
    torch.cuda.synchronize()
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    tol = TOL[dt]
    go, gl = host(out), host(lse).reshape(-1, q_len)
    errs = {"out": assert_close("out", go, f["out"][:, pos:], tol),
            "lse": assert_close("lse", gl, f["lse"][:, pos:], tol),
            "k_rows": assert_close("k_rows", host(kc[:, pos:]), f["yk"][:, pos:], tol)}
    print(w.name, {k: f"{e:.2e}" for k, e in errs.items()})


# Per-sequence cache lengths (xattn_decode_varlen): the sequences of one batch sit at
# different positions.  Qwen3-shaped heads (32 query heads, 8 KV heads, hd 128, bf16), four
# new tokens per step, so each KV head holds 16 query rows (two row chunks).
QWEN_HEADS = dict(num_heads=32, num_kv_heads=8, head_dim=128, theta=1e6, eps=1e-6)


def _varlen_inputs(prefill, steps, q_len, index, dtype="bf16", heads=QWEN_HEADS):
    B = len(prefill)
    S = max(prefill) + steps * q_len
    w = R(dtype, heads["head_dim"], S, B, heads["num_heads"], heads["num_kv_heads"],
          theta=heads["theta"], eps=heads["eps"], index=index)
    return w, W.make_inputs(w)


def _gather_rows(a, heads, starts, n):
    """[B*heads, S, hd] -> rows starts[b] .. starts[b] + n of every sequence b."""
    return np.concatenate([a[b * heads:(b + 1) * heads, p:p + n] for b, p in enumerate(starts)])


def _varlen_stepwise(w, x, prefill, steps, q_len, cap):
    H, Hkv, hd, dt = w.num_heads, w.num_kv_heads, w.head_dim, w.dtype
    cos, sin = X.rope_cache(cap, hd, w.theta)
    gq, gk = dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32")
    kc = torch.zeros((w.bkv, cap, hd), dtype=TDT[dt], device="cuda")
    vc = torch.zeros_like(kc)
    for b, p in enumerate(prefill):  # prefill sequence b's cache with its first p tokens
        if p:
            rows = slice(b * Hkv, (b + 1) * Hkv)
            yk, _ = X.qknorm_rope_fwd(dev(x.xk[rows, :p], dt), gk, cos, sin, w.eps)
            kc[rows, :p] = yk
            vc[rows, :p] = dev(x.v[rows, :p], dt)
    outs, lses = [], []
    for t in range(steps):
        pos = [p + t * q_len for p in prefill]
        lens = torch.tensor(pos, dtype=torch.int32, device="cuda")
        o, l = X.decode(dev(_gather_rows(x.xq, H, pos, q_len), dt),
                        dev(_gather_rows(x.xk, Hkv, pos, q_len), dt),
                        dev(_gather_rows(x.v, Hkv, pos, q_len), dt),
                        gq, gk, cos, sin, w.eps, kc, vc, lens, H, Hkv)
        outs.append(o)
        lses.append(l.reshape(-1, q_len))
    torch.cuda.synchronize()
    return (host(torch.cat(outs, dim=1)), host(torch.cat(lses, dim=1)), host(kc), host(vc))


def test_varlen_decode_matches_full_sequences():
    """Four sequences prefilled to 0, 13, 50 and 101 tokens, then eight decode steps of four
    tokens each: every decoded row equals the oracle's full-sequence forward."""
    prefill, steps, q_len = [0, 13, 50, 101], 8, 4
    w, x = _varlen_inputs(prefill, steps, q_len, 420)
    cap = w.seq_len + 7
    note(f"varlen decode stepwise prefill={prefill} steps={steps} q_len={q_len}")
    out, lse, kc, vc = _varlen_stepwise(w, x, prefill, steps, q_len, cap)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    n = steps * q_len
    H, Hkv = w.num_heads, w.num_kv_heads
    tol = TOL["bf16"]
    errs = {"out": assert_close("out", out, _gather_rows(f["out"], H, prefill, n), tol),
            "lse": assert_close("lse", lse, _gather_rows(f["lse"][..., None], H, prefill, n)[..., 0],
                                tol)}
    for b, p in enumerate(prefill):
        rows, end = slice(b * Hkv, (b + 1) * Hkv), p + n
        errs[f"k_cache{b}"] = assert_close(f"k_cache{b}", kc[rows, :end], f["yk"][rows, :end], tol)
        np.testing.assert_array_equal(vc[rows, :end], x.v[rows, :end].astype(np.float64))
        assert not kc[rows, end:].any() and not vc[rows, end:].any()  # rows past: untouched
    print({k: f"{e:.2e}" for k, e in errs.items()})
    again = _varlen_stepwise(w, x, prefill, steps, q_len, cap)
    for u, v in zip((out, lse, kc, vc), again):
        np.testing.assert_array_equal(u, v)  # bitwise reproducible


# The other split kernels with per-sequence lengths: fp32 (VALU), bf16 hd 64 (matrix cores),
# bf16 hd 16 / 32 (dot2), with row chunks where group * q_len passes one wave's rows.
VARLEN_KERNELS = [
    ("f32", dict(num_heads=8, num_kv_heads=2, head_dim=64, theta=1e4, eps=1e-5), [0, 9, 30], 3, 2),
    ("bf16", dict(num_heads=12, num_kv_heads=4, head_dim=64, theta=1e4, eps=1e-6), [5, 0, 41], 4, 3),
    ("bf16", dict(num_heads=16, num_kv_heads=2, head_dim=32, theta=1e6, eps=1e-6), [17, 3], 3, 4),
    ("f32", dict(num_heads=4, num_kv_heads=2, head_dim=16, theta=1e4, eps=1e-5), [0, 7, 2, 19], 5, 3),
]


@pytest.mark.parametrize("dt,heads,prefill,steps,q_len", VARLEN_KERNELS,
                         ids=[f"{v[0]}_hd{v[1]['head_dim']}_g{v[1]['num_heads'] // v[1]['num_kv_heads']}"
                              f"_q{v[4]}" for v in VARLEN_KERNELS])
def test_varlen_decode_other_kernels_match_full_sequences(dt, heads, prefill, steps, q_len):
    w, x = _varlen_inputs(prefill, steps, q_len, 430 + len(prefill), dt, heads)
    cap = w.seq_len + 3
    note(f"varlen decode {dt} {heads} prefill={prefill} steps={steps} q_len={q_len}")
    out, lse, kc, vc = _varlen_stepwise(w, x, prefill, steps, q_len, cap)
    f = oracle.forward(x.xq, x.xk, x.v, x.gamma_q, x.gamma_k, w.num_heads, w.num_kv_heads,
                       w.eps, w.theta)
    n = steps * q_len
    H, Hkv = w.num_heads, w.num_kv_heads
    tol = TOL[dt]
    assert_close("out", out, _gather_rows(f["out"], H, prefill, n), tol)
    assert_close("lse", lse, _gather_rows(f["lse"][..., None], H, prefill, n)[..., 0], tol)
    for b, p in enumerate(prefill):
        rows, end = slice(b * Hkv, (b + 1) * Hkv), p + n
        assert_close(f"k_cache{b}", kc[rows, :end], f["yk"][rows, :end], tol)
        np.testing.assert_array_equal(vc[rows, :end], x.v[rows, :end].astype(np.float64))
        assert not kc[rows, end:].any() and not vc[rows, end:].any()


def test_full_size_varlen_decode_mixed_cache_lengths():
    """A 4096-row cache per sequence holding seeded cache contents; the sequences hold 0, 1021,
    2900 and 4092 tokens and each decodes four more, compared per sequence with the oracle's
    decode step.  Cache rows past each sequence's new tokens hold values that would change
    the result if they were read, and must be left as they were."""
    lens, q_len, cap = [0, 1021, 2900, 4092], 4, 4096
    B = len(lens)
    H, Hkv, hd = QWEN_HEADS["num_heads"], QWEN_HEADS["num_kv_heads"], QWEN_HEADS["head_dim"]
    eps, theta = QWEN_HEADS["eps"], QWEN_HEADS["theta"]
    w = R("bf16", hd, q_len, B, H, Hkv, theta=theta, eps=eps, index=421)
    x = W.make_inputs(w)
    rng = np.random.default_rng(422)
    k0 = W.bf16_round(rng.standard_normal((B * Hkv, cap, hd), dtype=np.float32))
    v0 = W.bf16_round(rng.standard_normal((B * Hkv, cap, hd), dtype=np.float32))
    note(f"varlen decode full size lens={lens} q_len={q_len} cap={cap}")
    cos, sin = X.rope_cache(cap, hd, theta)
    runs = []
    for _ in range(2):
        kc, vc = dev(k0, "bf16"), dev(v0, "bf16")
        o, l = X.decode(dev(x.xq, "bf16"), dev(x.xk, "bf16"), dev(x.v, "bf16"),
                        dev(x.gamma_q, "f32"), dev(x.gamma_k, "f32"), cos, sin, eps, kc, vc,
                        torch.tensor(lens, dtype=torch.int32, device="cuda"), H, Hkv)
        torch.cuda.synchronize()
        runs.append((host(o), host(l).reshape(-1, q_len), host(kc), host(vc)))
    for u, v in zip(*runs):
        np.testing.assert_array_equal(u, v)  # bitwise reproducible
    out, lse, kc, vc = runs[0]
    tol = TOL["bf16"]
    for b, p in enumerate(lens):
        qs, ks = slice(b * H, (b + 1) * H), slice(b * Hkv, (b + 1) * Hkv)
        ro, rl, rk, rv = oracle.decode(x.xq[qs], x.xk[ks], x.v[ks], x.gamma_q, x.gamma_k,
                                       k0[ks], v0[ks], p, H, Hkv, eps, theta)
        errs = {"out": assert_close(f"out{b}", out[qs], ro, tol),
                "lse": assert_close(f"lse{b}", lse[qs], rl, tol),
                "k_rows": assert_close(f"k_rows{b}", kc[ks, p:p + q_len], rk[:, p:], tol)}
        np.testing.assert_array_equal(vc[ks, p:p + q_len], rv[:, p:])
        for c, c0 in ((kc, k0), (vc, v0)):  # every other cache row as it was
            np.testing.assert_array_equal(c[ks, :p], c0[ks, :p])
            np.testing.assert_array_equal(c[ks, p + q_len:], c0[ks, p + q_len:])
        print(b, p, {k: f"{e:.2e}" for k, e in errs.items()})
