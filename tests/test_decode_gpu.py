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
