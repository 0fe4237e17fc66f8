"""Scalar brute-force oracle (TEST INFRASTRUCTURE; same import rules as
oracle.py).  Pure-Python loops over every index, with the math module only, for
tiny shapes: it checks the vectorised oracle's indexing, masking, head mapping
and group sums element by element.  Formulas as in oracle.py (Mint docs 5.3.1,
5.4.1-5.4.4, 5.5.1-5.5.2; Phase T15 head mapping and group sum)."""
from __future__ import annotations

import math


def _rows(a):
    return [[list(map(float, row)) for row in head] for head in a]


def forward(xq, xk, v, gq, gk, H, Hkv, eps, theta):
    xq, xk, v = _rows(xq), _rows(xk), _rows(v)
    gq, gk = list(map(float, gq)), list(map(float, gk))
    BH, S, hd = len(xq), len(xq[0]), len(xq[0][0])
    half = hd // 2
    group = H // Hkv

    def prologue(x, g):
        y, rs = [], []
        for head in x:
            yh, rh = [], []
            for t, row in enumerate(head):
                ms = sum(e * e for e in row) / hd
                r = 1.0 / math.sqrt(ms + eps)
                n = [row[i] * r * g[i] for i in range(hd)]
                o = [0.0] * hd
                for i in range(half):
                    a = t * theta ** (-2.0 * i / hd)
                    c, s = math.cos(a), math.sin(a)
                    o[i] = n[i] * c - n[i + half] * s
                    o[i + half] = n[i] * s + n[i + half] * c
                yh.append(o)
                rh.append(r)
            y.append(yh)
            rs.append(rh)
        return y, rs

    yq, rq = prologue(xq, gq)
    yk, rk = prologue(xk, gk)
    out = [[[0.0] * hd for _ in range(S)] for _ in range(BH)]
    lse = [[0.0] * S for _ in range(BH)]
    probs = {}
    scale = 1.0 / math.sqrt(hd)
    for bh in range(BH):
        b, qh = divmod(bh, H)
        kv = b * Hkv + qh // group
        for i in range(S):
            s = [sum(yq[bh][i][d] * yk[kv][j][d] for d in range(hd)) * scale
                 for j in range(i + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            l = sum(e)
            p = [x / l for x in e]
            probs[(bh, i)] = p
            lse[bh][i] = m + math.log(l)
            for d in range(hd):
                out[bh][i][d] = sum(p[j] * v[kv][j][d] for j in range(i + 1))
    return dict(yq=yq, yk=yk, rstd_q=rq, rstd_k=rk, out=out, lse=lse, probs=probs)


def backward(xq, xk, v, gq, gk, dout, H, Hkv, eps, theta):
    f = forward(xq, xk, v, gq, gk, H, Hkv, eps, theta)
    xq, xk, v, dout = _rows(xq), _rows(xk), _rows(v), _rows(dout)
    gq, gk = list(map(float, gq)), list(map(float, gk))
    BH, S, hd = len(xq), len(xq[0]), len(xq[0][0])
    BKV = len(xk)
    half = hd // 2
    group = H // Hkv
    scale = 1.0 / math.sqrt(hd)
    yq, yk = f["yq"], f["yk"]
    dyq = [[[0.0] * hd for _ in range(S)] for _ in range(BH)]
    dyk = [[[0.0] * hd for _ in range(S)] for _ in range(BKV)]
    dv = [[[0.0] * hd for _ in range(S)] for _ in range(BKV)]
    for kv in range(BKV):
        b, kvh = divmod(kv, Hkv)
        for r in range(group):
            bh = b * H + kvh * group + r
            for i in range(S):
                p = f["probs"][(bh, i)]
                dp = [sum(dout[bh][i][d] * v[kv][j][d] for d in range(hd))
                      for j in range(i + 1)]
                D = sum(p[j] * dp[j] for j in range(i + 1))
                for j in range(i + 1):
                    ds = p[j] * (dp[j] - D)
                    for d in range(hd):
                        dyq[bh][i][d] += ds * yk[kv][j][d] * scale
                        dyk[kv][j][d] += ds * yq[bh][i][d] * scale
                        dv[kv][j][d] += p[j] * dout[bh][i][d]

    def prologue_bwd(dy, x, g, rstd):
        dx = [[[0.0] * hd for _ in range(S)] for _ in range(len(x))]
        dg = [0.0] * hd
        for h in range(len(x)):
            for t in range(S):
                dn = [0.0] * hd
                for i in range(half):
                    a = t * theta ** (-2.0 * i / hd)
                    c, s = math.cos(a), math.sin(a)
                    dn[i] = dy[h][t][i] * c + dy[h][t][i + half] * s
                    dn[i + half] = -dy[h][t][i] * s + dy[h][t][i + half] * c
                r = rstd[h][t]
                dot = sum(g[i] * dn[i] * x[h][t][i] for i in range(hd))
                for i in range(hd):
                    dx[h][t][i] = g[i] * dn[i] * r - x[h][t][i] * dot * r ** 3 / hd
                    dg[i] += dn[i] * x[h][t][i] * r
        return dx, dg

    dxq, dgq = prologue_bwd(dyq, xq, gq, f["rstd_q"])
    dxk, dgk = prologue_bwd(dyk, xk, gk, f["rstd_k"])
    return dict(dyq=dyq, dyk=dyk, dxq=dxq, dxk=dxk, dv=dv, dgamma_q=dgq, dgamma_k=dgk)
