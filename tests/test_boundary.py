"""Host-side checks of the C-ABI boundary: the library loads, exports every entry point
include/xattn.h declares, and rejects every invalid argument with the documented status
before touching the device.  No call here reaches a kernel launch (no GPU needed): each
one fails validation first."""
import ctypes
import os
import re

import pytest

import causal_gqa_attention_amd as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xattn.h")

OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
A = 0x10000  # a 16-byte aligned fake device address; never dereferenced
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(X.library_path()):
        pytest.fail("libxattn.so is not built (run python -m causal_gqa_attention_amd.build)")
    return X.load_library()


def test_library_exports_every_declared_entry_point(lib):
    names = declared_functions()
    assert len(names) == 25, names
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in X.xattn_version()


def test_status_strings(lib):
    for s in (OK, INVALID, UNSUPPORTED, HIPERR):
        assert lib.xattn_status_string(s).decode().startswith(
            ["XATTN_OK", "XATTN_ERR_INVALID_ARG", "XATTN_ERR_UNSUPPORTED", "XATTN_ERR_HIP"][s])
    assert "unknown" in lib.xattn_status_string(99).decode()


def dims(B=2, S=64, H=8, Hkv=2, hd=64, dt=1):
    return X.Dims(B, S, H, Hkv, hd, dt)


def fwd(lib, d, q=A, k=A + 8 * MB, v=A + 16 * MB, out=A + 24 * MB, lse=A + 32 * MB):
    return lib.xattn_fwd(ctypes.byref(d), q, k, v, out, lse, None)


def last(lib):
    return lib.xattn_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=6, Hkv=4), INVALID, "multiple of num_kv_heads"),
    (dict(Hkv=0), INVALID, "num_kv_heads"),
    (dict(B=0), INVALID, "batch"),
    (dict(S=-3), INVALID, "seq_len"),
    (dict(hd=63), INVALID, "even"),
    (dict(hd=48), UNSUPPORTED, "not supported"),
    (dict(hd=256), UNSUPPORTED, "not supported"),
    (dict(dt=7), INVALID, "dtype"),
    (dict(B=1 << 20, S=1 << 12, H=8, Hkv=8, hd=128), INVALID, "int32"),
])
def test_fwd_rejects_bad_dims(lib, kw, status, msg):
    assert fwd(lib, dims(**kw)) == status
    assert msg in last(lib)


def test_fwd_rejects_null_and_misaligned_pointers(lib):
    d = dims()
    assert fwd(lib, d, q=None) == INVALID and "q is NULL" in last(lib)
    assert fwd(lib, d, lse=None) == INVALID and "lse is NULL" in last(lib)
    assert fwd(lib, d, v=A + 8 * MB + 16 * MB + 2) == INVALID and "aligned" in last(lib)
    assert lib.xattn_fwd(None, A, A, A, A, A, None) == INVALID and "dims" in last(lib)


def test_fwd_rejects_aliasing_outputs(lib):
    d = dims()
    assert fwd(lib, d, out=A) == INVALID and "overlaps input q" in last(lib)
    assert fwd(lib, d, lse=A + 24 * MB + 4096) == INVALID and "overlap" in last(lib)


def test_prologue_fwd_validation(lib):
    f = lib.xattn_qknorm_rope_fwd
    base = [A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB]
    assert f(None, *base[1:], 4, 16, 64, 1e-5, 0, None) == INVALID
    assert f(*base, 4, 16, 64, -1.0, 0, None) == INVALID and "eps" in last(lib)
    assert f(*base, 4, 16, 64, float("nan"), 0, None) == INVALID
    assert f(*base, 4, 16, 60, 1e-5, 0, None) == UNSUPPORTED
    assert f(*base, 0, 16, 64, 1e-5, 0, None) == INVALID and "rows" in last(lib)
    # y overlapping x
    assert f(A, base[1], base[2], base[3], A + 64, base[5], 4, 16, 64, 1e-5, 0, None) == INVALID


def fwd_qnorm(lib, d, pro, k=A + 40 * MB, v=A + 48 * MB, out=A + 56 * MB, lse=A + 64 * MB):
    return lib.xattn_fwd_qnorm(ctypes.byref(d), ctypes.byref(pro) if pro is not None else None,
                               k, v, out, lse, None)


def test_fwd_qnorm_validation(lib):
    d = dims()  # bf16, B=2, S=64, H=8, hd=64: every tensor is well under 8 MiB
    good = dict(xq=A, gamma_q=A + 8 * MB, cos_tab=A + 9 * MB, sin_tab=A + 10 * MB, eps=1e-5,
                yq=A + 16 * MB, rstd_q=A + 24 * MB)
    pro = lambda **kw: X.FwdPrologue(**{**good, **kw})
    assert fwd_qnorm(lib, d, None) == INVALID and "pro is NULL" in last(lib)
    assert fwd_qnorm(lib, d, pro(xq=None)) == INVALID and "pro->xq is NULL" in last(lib)
    assert fwd_qnorm(lib, d, pro(eps=-1.0)) == INVALID and "eps" in last(lib)
    assert fwd_qnorm(lib, d, pro(eps=float("nan"))) == INVALID and "eps" in last(lib)
    assert fwd_qnorm(lib, d, pro(yq=A + 64)) == INVALID and "overlaps input pro->xq" in last(lib)
    assert fwd_qnorm(lib, d, pro(rstd_q=A + 56 * MB)) == INVALID and "overlap" in last(lib)
    assert fwd_qnorm(lib, d, pro(), k=A + 8 * MB + 2) == INVALID and "aligned" in last(lib)
    assert fwd_qnorm(lib, dims(hd=48), pro()) == UNSUPPORTED


def ddims(B=2, H=8, Hkv=2, hd=64, dt=1, q_len=1, cache_len=10, cap=64):
    return X.DecodeDims(B, H, Hkv, hd, dt, q_len, cache_len, cap)


def decode_call(lib, d, eps=1e-5, ws_bytes=None, **kw):
    # every tensor of ddims() is well under 1 MiB; 1 MiB apart each
    names = ["xq", "xk", "v", "gamma_q", "gamma_k", "cos_tab", "sin_tab", "k_cache", "v_cache",
             "out", "lse", "workspace"]
    p = {n: A + i * MB for i, n in enumerate(names)}
    p.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.xattn_decode_workspace_bytes(ctypes.byref(d))
    return lib.xattn_decode(ctypes.byref(d), p["xq"], p["xk"], p["v"], p["gamma_q"],
                            p["gamma_k"], p["cos_tab"], p["sin_tab"], eps, p["k_cache"],
                            p["v_cache"], p["out"], p["lse"], p["workspace"], ws_bytes, None)


def test_decode_workspace_query(lib):
    w = [lib.xattn_decode_workspace_bytes(ctypes.byref(ddims(cache_len=c))) for c in (0, 10, 63)]
    assert w[0] > 0 and w[0] == w[1] == w[2]  # sized by capacity, not by cache_len
    assert lib.xattn_decode_workspace_bytes(ctypes.byref(ddims(cache_len=64))) == 0
    assert lib.xattn_decode_workspace_bytes(None) == 0


def test_decode_validation(lib):
    assert decode_call(lib, ddims(cache_len=64), ws_bytes=1 << 20) == INVALID
    assert "exceeds capacity" in last(lib)
    assert decode_call(lib, ddims(cache_len=-1), ws_bytes=1 << 20) == INVALID
    assert "cache_len" in last(lib)
    assert decode_call(lib, ddims(q_len=0), ws_bytes=1 << 20) == INVALID and "q_len" in last(lib)
    assert decode_call(lib, ddims(H=6, Hkv=4), ws_bytes=1 << 20) == INVALID
    assert decode_call(lib, ddims(hd=48), ws_bytes=1 << 20) == UNSUPPORTED
    assert decode_call(lib, ddims(), eps=-1.0) == INVALID and "eps" in last(lib)
    assert decode_call(lib, ddims(), xq=None) == INVALID and "xq is NULL" in last(lib)
    assert decode_call(lib, ddims(), lse=A + 10 * MB + 4) == INVALID and "aligned" in last(lib)
    d = ddims()
    ws = lib.xattn_decode_workspace_bytes(ctypes.byref(d))
    assert decode_call(lib, d, ws_bytes=ws - 1) == INVALID and "workspace too small" in last(lib)
    assert decode_call(lib, d, out=A) == INVALID and "overlaps input xq" in last(lib)
    assert decode_call(lib, d, v_cache=A + 7 * MB + 256) == INVALID and "overlap" in last(lib)


@pytest.mark.parametrize("dt,q_len", [(1, 3), (1, 16), (0, 5), (0, 48)])
def test_decode_any_rows_per_kv_head(lib, dt, q_len):
    # group * q_len beyond one wave's rows (8 bf16, 16 fp32) passes the shape checks and
    # fails only on the workspace size (given too small on purpose), before any launch
    d = ddims(dt=dt, q_len=q_len)
    assert decode_call(lib, d, ws_bytes=16) == INVALID and "workspace too small" in last(lib)


def test_decode_varlen_validation(lib):
    def call(d, cache_lens, **kw):
        names = ["xq", "xk", "v", "gamma_q", "gamma_k", "cos_tab", "sin_tab", "k_cache",
                 "v_cache", "out", "lse", "workspace"]
        p = {n: A + i * MB for i, n in enumerate(names)}
        p.update(kw)
        ws = lib.xattn_decode_workspace_bytes(ctypes.byref(d))
        return lib.xattn_decode_varlen(
            ctypes.byref(d), cache_lens, p["xq"], p["xk"], p["v"], p["gamma_q"], p["gamma_k"],
            p["cos_tab"], p["sin_tab"], 1e-5, p["k_cache"], p["v_cache"], p["out"], p["lse"],
            p["workspace"], ws, None)
    assert call(ddims(), None) == INVALID and "cache_lens is NULL" in last(lib)
    assert call(ddims(), A + 20 * MB + 4) == INVALID and "aligned" in last(lib)
    assert call(ddims(), A + 20 * MB, lse=A + 20 * MB) == INVALID
    assert "overlaps input cache_lens" in last(lib)
    assert call(ddims(cache_len=64), A + 20 * MB) == INVALID and "exceeds capacity" in last(lib)


def test_document_arrays_validation(lib):
    d = dims()
    d.seg_lo = A + 40 * MB
    assert fwd(lib, d) == INVALID and "both be set" in last(lib)
    d.seg_hi = A + 40 * MB + 4  # misaligned
    assert fwd(lib, d) == INVALID and "aligned" in last(lib)
    d.seg_hi = A + 48 * MB
    assert fwd(lib, d, out=A + 40 * MB) == INVALID and "overlaps input seg_lo" in last(lib)


def test_segments_and_rope_table_at_validation(lib):
    f = lib.xattn_segments
    assert f(None, 2, 16, A, A + MB, A + 2 * MB, None) == INVALID and "cu_seqlens" in last(lib)
    assert f(A, 0, 16, A + MB, A + 2 * MB, None, None) == INVALID and "ndocs" in last(lib)
    assert f(A, 17, 16, A + MB, A + 2 * MB, None, None) == INVALID and "exceeds" in last(lib)
    assert f(A, 2, 16, A + MB, A + MB + 32, None, None) == INVALID and "overlap" in last(lib)
    assert f(A, 2, 16, A, A + MB, None, None) == INVALID and "overlaps input" in last(lib)
    g = lib.xattn_rope_cache_at
    assert g(A, A + MB, None, 16, 64, 1e4, None) == INVALID and "positions" in last(lib)
    assert g(A, A + MB, A + 2 * MB, 16, 64, -1.0, None) == INVALID and "theta" in last(lib)
    assert g(A, A + MB, A + 2 * MB, 16, 48, 1e4, None) == UNSUPPORTED
    assert g(A, A + MB, A, 16, 64, 1e4, None) == INVALID and "overlaps input" in last(lib)


def test_projection_validation(lib):
    d = dims()  # B=2, S=64, H=8, Hkv=2, hd=64, bf16
    ws = lib.xattn_proj_workspace_bytes(ctypes.byref(d), 128)
    assert ws > 0
    assert lib.xattn_proj_workspace_bytes(ctypes.byref(d), 100) == 0  # d % 8 != 0
    assert "multiple of 8" in last(lib)
    p = X.Proj(128, A, A + MB, A + 2 * MB, A + 3 * MB, None, None, None, None)
    f = lib.xattn_qkv_proj_fwd
    io = [A + 4 * MB, A + 8 * MB, A + 12 * MB, A + 16 * MB]  # x, xq, xk, v
    assert f(ctypes.byref(d), None, *io, A + 32 * MB, ws, None) == INVALID and "p is NULL" in last(lib)
    assert f(ctypes.byref(d), ctypes.byref(p), *io, A + 32 * MB, ws - 1, None) == INVALID
    assert "workspace too small" in last(lib)
    assert f(ctypes.byref(d), ctypes.byref(p), None, *io[1:], A + 32 * MB, ws, None) == INVALID
    assert f(ctypes.byref(d), ctypes.byref(p), io[0], A, io[2], io[3], A + 32 * MB, ws,
             None) == INVALID and "overlaps input" in last(lib)
    p.bq = A + 3 * MB + 2
    assert f(ctypes.byref(d), ctypes.byref(p), *io, A + 32 * MB, ws, None) == INVALID
    assert "aligned" in last(lib)
    g = lib.xattn_out_proj_bwd
    p.bq = None
    assert g(ctypes.byref(d), ctypes.byref(p), A + 4 * MB, A + 8 * MB, A + 12 * MB, None, None,
             A + 32 * MB, ws, None) == INVALID and "dwo is NULL" in last(lib)


def test_rope_cache_validation(lib):
    f = lib.xattn_rope_cache
    assert f(A, A + MB, 16, 64, 0.0, None) == INVALID and "theta" in last(lib)
    assert f(A, A + MB, 16, 64, float("inf"), None) == INVALID
    assert f(A, A + MB, 0, 64, 1e4, None) == INVALID
    assert f(A, A + 8, 16, 64, 1e4, None) == INVALID  # tables overlap
    assert f(A, None, 16, 64, 1e4, None) == INVALID


def test_prologue_fwd_table_validation(lib):
    f = lib.xattn_qknorm_rope_fwd_table
    # x, gamma, positions, theta, cos, sin, y, rstd, rows, S, hd, eps, dtype, stream
    x, g, cs, sn, y, r = A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB
    assert f(None, g, None, 1e4, cs, sn, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID
    assert f(x, g, None, 0.0, cs, sn, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID
    assert "theta" in last(lib)
    assert f(x, g, None, 1e4, cs, sn, y, r, 4, 16, 64, -1.0, 0, None) == INVALID
    assert "eps" in last(lib)
    assert f(x, g, None, 1e4, cs, sn, y, r, 4, 16, 48, 1e-5, 0, None) == UNSUPPORTED
    assert f(x, g, None, 1e4, cs, sn, y, r, 4, 0, 64, 1e-5, 0, None) == INVALID
    assert f(x, g, A + 6 * MB + 2, 1e4, cs, sn, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID
    # the table is an output: it may not overlap x, another output or the positions
    assert f(x, g, None, 1e4, x + 64, sn, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID
    assert f(x, g, None, 1e4, cs, cs + 8, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID
    assert f(x, g, sn, 1e4, cs, sn, y, r, 4, 16, 64, 1e-5, 0, None) == INVALID


def test_prologue_bwd_workspace_and_validation(lib):
    ws = lib.xattn_qknorm_rope_bwd_workspace_bytes(1024, 1024, 64)
    assert ws > 0 and ws % (64 * 4) == 0
    assert lib.xattn_qknorm_rope_bwd_workspace_bytes(0, 1, 64) == 0
    f = lib.xattn_qknorm_rope_bwd
    p = [A + i * 64 * MB for i in range(9)]
    assert f(*p, ws - 4, 1024, 1024, 64, 1, None) == INVALID and "workspace too small" in last(lib)
    assert f(*p[:8], None, ws, 1024, 1024, 64, 1, None) == INVALID


def test_bwd_workspace_and_validation(lib):
    d = dims()
    w0 = lib.xattn_bwd_workspace_bytes(ctypes.byref(d), 0)
    w1 = lib.xattn_bwd_workspace_bytes(ctypes.byref(d), 1)
    assert w0 >= 2 * 8 * 64 * 4 and w1 > w0
    bad = dims(H=6, Hkv=4)
    assert lib.xattn_bwd_workspace_bytes(ctypes.byref(bad), 0) == 0
    p = [A + i * 16 * MB for i in range(10)]
    f = lib.xattn_bwd
    assert f(ctypes.byref(d), *p[:9], None, p[9], w0 - 1, None) == INVALID
    assert "workspace too small" in last(lib)
    assert f(ctypes.byref(d), *p[:9], None, None, w0, None) == INVALID
    # dq aliasing dout
    assert f(ctypes.byref(d), *p[:6], p[5], p[7], p[8], None, p[9], w0, None) == INVALID
    # prologue with a NULL member
    pro = X.Prologue(*[A + (20 + i) * 16 * MB for i in range(10)])
    pro.rstd_k = None
    assert f(ctypes.byref(d), *p[:9], ctypes.byref(pro), p[9], w1, None) == INVALID
    assert "rstd_k" in last(lib)


def test_profile_stop_validation_and_empty_session(lib):
    n = ctypes.c_int32(-1)
    assert lib.xattn_profile_stop(None, 4, ctypes.byref(n)) == INVALID
    assert lib.xattn_profile_stop(None, 0, None) == INVALID
    # a session with no launches reports no kernels (no device work involved)
    assert lib.xattn_profile_start() == OK
    assert lib.xattn_profile_stop(None, 0, ctypes.byref(n)) == OK and n.value == 0


def test_python_binding_fails_loudly_without_device_tensors():
    import torch
    q, k = torch.zeros(16, 8, 64), torch.zeros(4, 8, 64)
    with pytest.raises(ValueError, match="device tensor"):
        X.attn_fwd(q, k, k, 8, 2)


# The binding checks every tensor's element count against the call's dimensions before it
# looks at placement: the C ABI receives raw pointers, so a short tensor would otherwise
# reach the kernels.  CPU tensors of the right sizes get as far as the placement check.
def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_checks_attention_tensor_sizes():
    import torch
    B, S, H, Hkv, hd = 2, 8, 4, 2, 64
    q, k = _cpu(B * H, S, hd), _cpu(B * Hkv, S, hd)
    lse = _cpu(B * H * S, dtype=torch.float32)
    d = X.make_dims(q, H, Hkv)
    with pytest.raises(ValueError, match="device tensor"):
        X.xattn_fwd(d, q, k, k, q.clone(), lse)
    short_k = _cpu(B * Hkv, S - 1, hd)
    with pytest.raises(ValueError, match="k must hold 2048 elements"):
        X.xattn_fwd(d, q, short_k, k, q.clone(), lse)
    with pytest.raises(ValueError, match="lse must hold 64 elements"):
        X.xattn_fwd(d, q, k, k, q.clone(), lse[:-1])
    with pytest.raises(ValueError, match="out must hold"):
        X.xattn_fwd(d, q, k, k, k.clone(), lse)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="dv must hold"):
        X.xattn_bwd(d, q, k, k, q, lse, q, q.clone(), k.clone(), q.clone(), None, ws)
    f32 = torch.float32
    pro = dict(xq=q, xk=k, gamma_q=_cpu(hd, dtype=f32), gamma_k=_cpu(hd, dtype=f32),
               rstd_q=_cpu(B * H * S, dtype=f32), rstd_k=_cpu(B * Hkv * S, dtype=f32),
               cos_tab=_cpu(S, hd // 2, dtype=f32), sin_tab=_cpu(S - 1, hd // 2, dtype=f32),
               dgamma_q=_cpu(hd, dtype=f32), dgamma_k=_cpu(hd, dtype=f32))
    with pytest.raises(ValueError, match="sin_tab must hold at least 256 elements"):
        X.xattn_bwd(d, q, k, k, q, lse, q, q.clone(), k.clone(), k.clone(), pro, ws)
    pro["sin_tab"] = pro["cos_tab"].clone()
    pro["rstd_k"] = _cpu(B * H * S, dtype=f32)  # sized like rstd_q: wrong
    with pytest.raises(ValueError, match="rstd_k must hold 32 elements"):
        X.xattn_bwd(d, q, k, k, q, lse, q, q.clone(), k.clone(), k.clone(), pro, ws)
    with pytest.raises(ValueError, match="rstd_q must hold"):
        X.xattn_fwd_qnorm(d, q, pro["gamma_q"], pro["cos_tab"], pro["sin_tab"], 1e-5, q.clone(),
                          lse[:8], k, k, q.clone(), lse)
    seg = _cpu(S - 2, dtype=torch.int32)
    with pytest.raises(ValueError, match="seg_lo must hold 8 elements"):
        X.make_dims(q, H, Hkv, (seg, seg))


def test_binding_checks_prologue_and_table_sizes():
    import torch
    f32 = torch.float32
    rows, S, hd = 3, 10, 32
    x, g = _cpu(rows, S, hd), _cpu(hd, dtype=f32)
    cs, rs = _cpu(S, hd // 2, dtype=f32), _cpu(rows * S, dtype=f32)
    with pytest.raises(ValueError, match="cos_tab must hold at least 160 elements"):
        X.xattn_qknorm_rope_fwd(x, g, cs[:-1], cs, x.clone(), rs, rows, S, hd, 1e-5)
    with pytest.raises(ValueError, match="gamma must hold 32 elements"):
        X.xattn_qknorm_rope_fwd(x, g[:16], cs, cs, x.clone(), rs, rows, S, hd, 1e-5)
    with pytest.raises(ValueError, match="y must hold"):
        X.xattn_qknorm_rope_fwd(x, g, cs, cs, x[:2].clone(), rs, rows, S, hd, 1e-5)
    with pytest.raises(ValueError, match="positions must hold 10 elements"):
        X.xattn_qknorm_rope_fwd_table(x, g, _cpu(S + 1, dtype=torch.int32), 1e4, cs, cs,
                                      x.clone(), rs, rows, S, hd, 1e-5)
    with pytest.raises(ValueError, match="rstd must hold 30 elements"):
        X.xattn_qknorm_rope_bwd(x, x, g, rs[:-1], cs, cs, x.clone(), g.clone(),
                                torch.zeros(16, dtype=torch.uint8), rows, S, hd)
    with pytest.raises(ValueError, match="sin_tab must hold at least 64 elements"):
        X.xattn_rope_cache(_cpu(4, 16, dtype=f32), _cpu(3, 16, dtype=f32), 4, 32, 1e4)
    with pytest.raises(ValueError, match="positions must hold 5 elements"):
        X.xattn_rope_cache_at(_cpu(5, 16, dtype=f32), _cpu(5, 16, dtype=f32),
                              _cpu(4, dtype=torch.int32), 5, 32, 1e4)
    with pytest.raises(ValueError, match="cu_seqlens must hold 3 elements"):
        X.xattn_segments(_cpu(4, dtype=torch.int32), 2, 9, *(_cpu(9, dtype=torch.int32)
                                                              for _ in range(3)))


def test_binding_checks_decode_sizes():
    import torch
    f32 = torch.float32
    B, H, Hkv, hd, q_len, cap = 2, 8, 2, 128, 1, 40
    xq, xk = _cpu(B * H, q_len, hd), _cpu(B * Hkv, q_len, hd)
    kc = _cpu(B * Hkv, cap, hd)
    g, tab = _cpu(hd, dtype=f32), _cpu(cap, hd // 2, dtype=f32)
    with pytest.raises(ValueError, match="k_cache must be"):
        X.make_decode_dims(xq, _cpu(B * Hkv + 1, cap, hd), H, Hkv, 10)
    d = X.make_decode_dims(xq, kc, H, Hkv, 10)
    ws = torch.zeros(16, dtype=torch.uint8)
    lse = _cpu(B * H * q_len, dtype=f32)
    with pytest.raises(ValueError, match="cos_tab must hold at least 2560 elements"):
        X.xattn_decode(d, xq, xk, xk, g, g, tab[:-1], tab, 1e-6, kc, kc.clone(), xq.clone(),
                       lse, ws)
    with pytest.raises(ValueError, match="v_cache must hold"):
        X.xattn_decode(d, xq, xk, xk, g, g, tab, tab, 1e-6, kc, kc[:, :-1].clone(), xq.clone(),
                       lse, ws)
    with pytest.raises(ValueError, match="device tensor"):
        X.xattn_decode(d, xq, xk, xk, g, g, tab, tab, 1e-6, kc, kc.clone(), xq.clone(), lse, ws)


def test_bwd_noalloc_validation(lib):
    """Shapes beyond the static scratch and invalid dims are rejected before any device
    call."""
    big = dims(B=4, S=16384, H=64, Hkv=8, hd=128)
    assert lib.xattn_bwd_workspace_bytes(ctypes.byref(big), 0) > (16 << 20)
    p = [A + i * 16 * MB for i in range(9)]
    assert lib.xattn_bwd_noalloc(ctypes.byref(big), *p, None, None) == UNSUPPORTED
    assert "static scratch" in last(lib)
    assert lib.xattn_bwd_noalloc(ctypes.byref(dims(H=6, Hkv=4)), *p, None, None) == INVALID
    assert "multiple of num_kv_heads" in last(lib)
    assert lib.xattn_bwd_noalloc(None, *p, None, None) == INVALID
