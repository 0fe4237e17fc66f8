"""Python binding of libxattn: causal GQA attention with a QK-norm + RoPE prologue on
MI355X (gfx950).

This module only marshals arguments: it checks every tensor's element count against the
call's dimensions (the C ABI receives raw pointers and cannot), then its dtype, placement
and contiguity, allocates outputs and workspaces with torch (device memory and streams are
all torch is used for) and calls the C ABI declared in include/xattn.h.  Every computation runs in
the HIP kernels of libxattn.so; there is no fallback path.  If the library has not been
built, every call raises.

The functions named xattn_* mirror the C entry points one to one (same argument order,
torch tensors in place of device pointers).  The short helpers below them (rope_cache,
qknorm_rope_fwd, ...) allocate the outputs and call those.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "XattnError", "library_path", "load_library",
    "xattn_rope_cache", "xattn_qknorm_rope_fwd", "xattn_qknorm_rope_fwd_table",
    "xattn_qknorm_rope_bwd_workspace_bytes",
    "xattn_qknorm_rope_bwd", "xattn_fwd", "xattn_fwd_qnorm", "xattn_bwd_workspace_bytes",
    "xattn_bwd", "xattn_bwd_noalloc",
    "xattn_decode_workspace_bytes", "xattn_decode", "xattn_decode_varlen", "xattn_segments", "xattn_rope_cache_at",
    "xattn_proj_workspace_bytes", "xattn_qkv_proj_fwd", "xattn_out_proj_fwd",
    "xattn_out_proj_bwd", "xattn_qkv_proj_bwd",
    "xattn_status_string", "xattn_last_error", "xattn_version", "xattn_profile_start",
    "xattn_profile_stop",
    "rope_cache", "qknorm_rope_fwd", "qknorm_rope_fwd_table", "qknorm_rope_bwd", "attn_fwd", "attn_fwd_qnorm",
    "attn_bwd", "decode", "segments", "rope_cache_at", "Projection",
]

XATTN_F32 = 0
XATTN_BF16 = 1
_DTYPES = {torch.float32: XATTN_F32, torch.bfloat16: XATTN_BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class XattnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq_len", ctypes.c_int64),
                ("num_heads", ctypes.c_int64), ("num_kv_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("seg_lo", ctypes.c_void_p), ("seg_hi", ctypes.c_void_p)]


class Prologue(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("xk", ctypes.c_void_p),
                ("gamma_q", ctypes.c_void_p), ("gamma_k", ctypes.c_void_p),
                ("rstd_q", ctypes.c_void_p), ("rstd_k", ctypes.c_void_p),
                ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
                ("dgamma_q", ctypes.c_void_p), ("dgamma_k", ctypes.c_void_p)]


class FwdPrologue(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("gamma_q", ctypes.c_void_p),
                ("cos_tab", ctypes.c_void_p), ("sin_tab", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("yq", ctypes.c_void_p), ("rstd_q", ctypes.c_void_p)]


class Proj(ctypes.Structure):
    _fields_ = [("model_dim", ctypes.c_int64)] + [
        (n, ctypes.c_void_p) for n in ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo")]


class DecodeDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "num_heads", "num_kv_heads", "head_dim",
                                              "dtype", "q_len", "cache_len", "capacity")]


def library_path() -> str:
    return os.path.join(_HERE, "libxattn.so")


def load_library() -> ctypes.CDLL:
    """Load libxattn.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m causal_gqa_attention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sigs = {
        "xattn_rope_cache": (i32, [vp, vp, i64, i64, ctypes.c_double, vp]),
        "xattn_rope_cache_at": (i32, [vp, vp, vp, i64, i64, ctypes.c_double, vp]),
        "xattn_segments": (i32, [vp, i32, i64, vp, vp, vp, vp]),
        "xattn_qknorm_rope_fwd": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_float,
                                        i32, vp]),
        "xattn_qknorm_rope_fwd_table": (i32, [vp, vp, vp, ctypes.c_double, vp, vp, vp, vp, i64,
                                              i64, i64, ctypes.c_float, i32, vp]),
        "xattn_qknorm_rope_bwd_workspace_bytes": (sz, [i64, i64, i64]),
        "xattn_qknorm_rope_bwd": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, i64,
                                        i32, vp]),
        "xattn_fwd": (i32, [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp]),
        "xattn_fwd_qnorm": (i32, [ctypes.POINTER(Dims), ctypes.POINTER(FwdPrologue), vp, vp, vp,
                                  vp, vp]),
        "xattn_bwd_workspace_bytes": (sz, [ctypes.POINTER(Dims), ctypes.c_int]),
        "xattn_bwd": (i32, [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                            ctypes.POINTER(Prologue), vp, sz, vp]),
        "xattn_bwd_noalloc": (i32, [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    ctypes.POINTER(Prologue), vp]),
        "xattn_proj_workspace_bytes": (sz, [ctypes.POINTER(Dims), i64]),
        "xattn_qkv_proj_fwd": (i32, [ctypes.POINTER(Dims), ctypes.POINTER(Proj), vp, vp, vp,
                                     vp, vp, sz, vp]),
        "xattn_out_proj_fwd": (i32, [ctypes.POINTER(Dims), ctypes.POINTER(Proj), vp, vp, vp,
                                     sz, vp]),
        "xattn_out_proj_bwd": (i32, [ctypes.POINTER(Dims), ctypes.POINTER(Proj), vp, vp, vp,
                                     vp, vp, vp, sz, vp]),
        "xattn_qkv_proj_bwd": (i32, [ctypes.POINTER(Dims), ctypes.POINTER(Proj), vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "xattn_decode_workspace_bytes": (sz, [ctypes.POINTER(DecodeDims)]),
        "xattn_decode": (i32, [ctypes.POINTER(DecodeDims), vp, vp, vp, vp, vp, vp, vp,
                               ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]),
        "xattn_decode_varlen": (i32, [ctypes.POINTER(DecodeDims), vp, vp, vp, vp, vp, vp, vp,
                                      vp, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]),
        "xattn_profile_start": (i32, []),
        "xattn_profile_stop": (i32, [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]),
        "xattn_status_string": (ctypes.c_char_p, [i32]),
        "xattn_last_error": (ctypes.c_char_p, []),
        "xattn_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


# ----------------------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------------------
class AtLeast(int):
    """An element count that a tensor may exceed (a RoPE table with more rows than the call
    reads)."""


def _ptrs(*specs):
    """Device pointers of tensors given as (tensor, name, dtype, numel) specs, None entries
    passing through as NULL.  Every tensor is checked for its element count (numel, when
    not None: exactly, or at least for an AtLeast count; a shorter tensor would let the
    kernels read or write past it) and its dtype before any is checked for placement and
    contiguity, so a size mismatch is reported as such wherever the tensors live."""
    for t, name, dtype, numel in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if isinstance(numel, AtLeast) and t.numel() < numel:
            raise ValueError(f"{name} must hold at least {int(numel)} elements for these "
                             f"dimensions, got {t.numel()} (shape {tuple(t.shape)})")
        if numel is not None and not isinstance(numel, AtLeast) and t.numel() != int(numel):
            raise ValueError(f"{name} must hold {int(numel)} elements for these dimensions, "
                             f"got {t.numel()} (shape {tuple(t.shape)})")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    for t, name, _, _ in specs:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    return [None if t is None else t.data_ptr() for t, _, _, _ in specs]


def _bytes(t, name):
    """Size in bytes of a workspace tensor (the C side checks it against its query)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    return t.numel() * t.element_size()


def _sizes(dims):
    """Element counts of an attention call: (q / out / dout, k / v, lse / rstd_q rows,
    rstd_k rows, one rope table)."""
    B, S, H, Hkv, hd = dims.batch, dims.seq_len, dims.num_heads, dims.num_kv_heads, dims.head_dim
    return B * H * S * hd, B * Hkv * S * hd, B * H * S, B * Hkv * S, S * (hd // 2)


def _io(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name} must be float32 or bfloat16, got {t.dtype}")
    return _DTYPES[t.dtype]


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status, where):
    if status != 0:
        lib = load_library()
        detail = lib.xattn_last_error().decode() or lib.xattn_status_string(status).decode()
        raise XattnError(status, where, detail)


F32 = torch.float32
I32 = torch.int32


# ----------------------------------------------------------------------------------------
# one-to-one wrappers of the C entry points
# ----------------------------------------------------------------------------------------
def xattn_version() -> str:
    return load_library().xattn_version().decode()


def xattn_status_string(status: int) -> str:
    return load_library().xattn_status_string(status).decode()


def xattn_last_error() -> str:
    return load_library().xattn_last_error().decode()


def xattn_profile_start():
    _check(load_library().xattn_profile_start(), "xattn_profile_start")


def xattn_profile_stop(max_entries: int = 32) -> dict:
    """Returns {kernel name: (launches, total milliseconds)} in first-launch order."""
    entries = (KernelTime * max_entries)()
    n = ctypes.c_int32(0)
    _check(load_library().xattn_profile_stop(entries, max_entries, ctypes.byref(n)),
           "xattn_profile_stop")
    return {entries[i].name.decode(): (int(entries[i].launches), float(entries[i].total_ms))
            for i in range(min(n.value, max_entries))}


def xattn_rope_cache(cos_tab, sin_tab, seq_len, head_dim, theta, stream=None):
    nt = int(seq_len) * (int(head_dim) // 2)
    pc, ps = _ptrs((cos_tab, "cos_tab", F32, AtLeast(nt)),
                   (sin_tab, "sin_tab", F32, AtLeast(nt)))
    _check(load_library().xattn_rope_cache(pc, ps, seq_len, head_dim, float(theta),
                                           _stream(stream)), "xattn_rope_cache")


def _prologue_sizes(rows, seq_len, head_dim):
    return int(rows) * seq_len * head_dim, int(rows) * seq_len, seq_len * (head_dim // 2)


def xattn_qknorm_rope_fwd(x, gamma, cos_tab, sin_tab, y, rstd, rows, seq_len, head_dim, eps,
                          stream=None):
    n, nr, nt = _prologue_sizes(rows, seq_len, head_dim)
    io = _io(x, "x")
    p = _ptrs((x, "x", None, n), (gamma, "gamma", F32, head_dim),
              (cos_tab, "cos_tab", F32, AtLeast(nt)), (sin_tab, "sin_tab", F32, AtLeast(nt)),
              (y, "y", x.dtype, n), (rstd, "rstd", F32, nr))
    _check(load_library().xattn_qknorm_rope_fwd(*p, rows, seq_len, head_dim, float(eps), io,
                                                _stream(stream)), "xattn_qknorm_rope_fwd")


def xattn_qknorm_rope_fwd_table(x, gamma, positions, theta, cos_tab, sin_tab, y, rstd, rows,
                                seq_len, head_dim, eps, stream=None):
    n, nr, nt = _prologue_sizes(rows, seq_len, head_dim)
    io = _io(x, "x")
    px, pg, ppos, pc, ps, py, pr = _ptrs(
        (x, "x", None, n), (gamma, "gamma", F32, head_dim), (positions, "positions", I32, seq_len),
        (cos_tab, "cos_tab", F32, AtLeast(nt)), (sin_tab, "sin_tab", F32, AtLeast(nt)),
        (y, "y", x.dtype, n),
        (rstd, "rstd", F32, nr))
    _check(load_library().xattn_qknorm_rope_fwd_table(
        px, pg, ppos, float(theta), pc, ps, py, pr, rows, seq_len, head_dim, float(eps), io,
        _stream(stream)), "xattn_qknorm_rope_fwd_table")


def xattn_qknorm_rope_bwd_workspace_bytes(rows, seq_len, head_dim) -> int:
    return int(load_library().xattn_qknorm_rope_bwd_workspace_bytes(rows, seq_len, head_dim))


def xattn_qknorm_rope_bwd(dy, x, gamma, rstd, cos_tab, sin_tab, dx, dgamma, workspace, rows,
                          seq_len, head_dim, stream=None):
    n, nr, nt = _prologue_sizes(rows, seq_len, head_dim)
    io = _io(x, "x")
    p = _ptrs((dy, "dy", x.dtype, n), (x, "x", None, n), (gamma, "gamma", F32, head_dim),
              (rstd, "rstd", F32, nr), (cos_tab, "cos_tab", F32, AtLeast(nt)),
              (sin_tab, "sin_tab", F32, AtLeast(nt)), (dx, "dx", x.dtype, n),
              (dgamma, "dgamma", F32, head_dim), (workspace, "workspace", None, None))
    _check(load_library().xattn_qknorm_rope_bwd(
        *p, _bytes(workspace, "workspace"), rows, seq_len, head_dim, io, _stream(stream)),
        "xattn_qknorm_rope_bwd")


def make_dims(q, num_heads, num_kv_heads, segments=None) -> Dims:
    """q: [B*H, S, hd]; segments: None, or (seg_lo, seg_hi) int32 device tensors [S] (see
    xattn_segments)."""
    bh, S, hd = q.shape
    if bh % num_heads:
        raise ValueError("q.shape[0] must be batch * num_heads")
    lo = hi = None
    if segments is not None:
        lo, hi = _ptrs((segments[0], "seg_lo", I32, S), (segments[1], "seg_hi", I32, S))
    return Dims(bh // num_heads, S, num_heads, num_kv_heads, hd, _io(q, "q"), lo, hi)


def xattn_segments(cu_seqlens, ndocs, seq_len, seg_lo, seg_hi, positions=None, stream=None):
    S = int(seq_len)
    p = _ptrs((cu_seqlens, "cu_seqlens", I32, int(ndocs) + 1), (seg_lo, "seg_lo", I32, S),
              (seg_hi, "seg_hi", I32, S), (positions, "positions", I32, S))
    _check(load_library().xattn_segments(p[0], int(ndocs), S, *p[1:], _stream(stream)),
           "xattn_segments")


def xattn_rope_cache_at(cos_tab, sin_tab, positions, rows, head_dim, theta, stream=None):
    nt = int(rows) * (int(head_dim) // 2)
    p = _ptrs((cos_tab, "cos_tab", F32, AtLeast(nt)), (sin_tab, "sin_tab", F32, AtLeast(nt)),
              (positions, "positions", I32, rows))
    _check(load_library().xattn_rope_cache_at(*p, rows, head_dim, theta, _stream(stream)),
           "xattn_rope_cache_at")


def xattn_fwd(dims: Dims, q, k, v, out, lse, stream=None):
    nq, nk, nr, _, _ = _sizes(dims)
    _io(q, "q")
    p = _ptrs((q, "q", None, nq), (k, "k", q.dtype, nk), (v, "v", q.dtype, nk),
              (out, "out", q.dtype, nq), (lse, "lse", F32, nr))
    _check(load_library().xattn_fwd(ctypes.byref(dims), *p, _stream(stream)), "xattn_fwd")


def xattn_fwd_qnorm(dims: Dims, xq, gamma_q, cos_tab, sin_tab, eps, yq, rstd_q, k, v, out,
                    lse, stream=None):
    nq, nk, nr, _, nt = _sizes(dims)
    hd = dims.head_dim
    _io(xq, "xq")
    pxq, pg, pc, ps, pyq, pr, pk, pv, po, pl = _ptrs(
        (xq, "xq", None, nq), (gamma_q, "gamma_q", F32, hd),
        (cos_tab, "cos_tab", F32, AtLeast(nt)), (sin_tab, "sin_tab", F32, AtLeast(nt)),
        (yq, "yq", xq.dtype, nq), (rstd_q, "rstd_q", F32, nr),
        (k, "k", xq.dtype, nk), (v, "v", xq.dtype, nk), (out, "out", xq.dtype, nq),
        (lse, "lse", F32, nr))
    pro = FwdPrologue(pxq, pg, pc, ps, float(eps), pyq, pr)
    _check(load_library().xattn_fwd_qnorm(ctypes.byref(dims), ctypes.byref(pro), pk, pv, po, pl,
                                          _stream(stream)), "xattn_fwd_qnorm")


def xattn_bwd_workspace_bytes(dims: Dims, with_prologue: bool) -> int:
    return int(load_library().xattn_bwd_workspace_bytes(ctypes.byref(dims), int(with_prologue)))


def xattn_bwd(dims: Dims, q, k, v, out, lse, dout, dq, dk, dv, prologue, workspace,
              stream=None):
    """prologue: None or a dict with xq, xk, gamma_q, gamma_k, rstd_q, rstd_k, cos_tab,
    sin_tab, dgamma_q, dgamma_k tensors."""
    nq, nk, nr, nrk, nt = _sizes(dims)
    hd = dims.head_dim
    _io(q, "q")
    specs = [(q, "q", None, nq), (k, "k", q.dtype, nk), (v, "v", q.dtype, nk),
             (out, "out", q.dtype, nq), (lse, "lse", F32, nr), (dout, "dout", q.dtype, nq),
             (dq, "dq", q.dtype, nq), (dk, "dk", q.dtype, nk), (dv, "dv", q.dtype, nk),
             (workspace, "workspace", None, None)]
    if prologue is not None:
        pr = prologue
        specs += [(pr["xq"], "xq", q.dtype, nq), (pr["xk"], "xk", q.dtype, nk),
                  (pr["gamma_q"], "gamma_q", F32, hd), (pr["gamma_k"], "gamma_k", F32, hd),
                  (pr["rstd_q"], "rstd_q", F32, nr), (pr["rstd_k"], "rstd_k", F32, nrk),
                  (pr["cos_tab"], "cos_tab", F32, AtLeast(nt)),
                  (pr["sin_tab"], "sin_tab", F32, AtLeast(nt)),
                  (pr["dgamma_q"], "dgamma_q", F32, hd), (pr["dgamma_k"], "dgamma_k", F32, hd)]
    p = _ptrs(*specs)
    pro = Prologue(*p[10:]) if prologue is not None else None
    _check(load_library().xattn_bwd(
        ctypes.byref(dims), *p[:9], ctypes.byref(pro) if pro is not None else None, p[9],
        _bytes(workspace, "workspace"), _stream(stream)), "xattn_bwd")


def xattn_bwd_noalloc(dims: Dims, q, k, v, out, lse, dout, dq, dk, dv, prologue, stream=None):
    """xattn_bwd with the library's static scratch in place of a workspace (no allocation;
    calls that overlap on one GPU race on that scratch)."""
    nq, nk, nr, nrk, nt = _sizes(dims)
    hd = dims.head_dim
    _io(q, "q")
    specs = [(q, "q", None, nq), (k, "k", q.dtype, nk), (v, "v", q.dtype, nk),
             (out, "out", q.dtype, nq), (lse, "lse", F32, nr), (dout, "dout", q.dtype, nq),
             (dq, "dq", q.dtype, nq), (dk, "dk", q.dtype, nk), (dv, "dv", q.dtype, nk)]
    if prologue is not None:
        pr = prologue
        specs += [(pr["xq"], "xq", q.dtype, nq), (pr["xk"], "xk", q.dtype, nk),
                  (pr["gamma_q"], "gamma_q", F32, hd), (pr["gamma_k"], "gamma_k", F32, hd),
                  (pr["rstd_q"], "rstd_q", F32, nr), (pr["rstd_k"], "rstd_k", F32, nrk),
                  (pr["cos_tab"], "cos_tab", F32, AtLeast(nt)),
                  (pr["sin_tab"], "sin_tab", F32, AtLeast(nt)),
                  (pr["dgamma_q"], "dgamma_q", F32, hd), (pr["dgamma_k"], "dgamma_k", F32, hd)]
    p = _ptrs(*specs)
    pro = Prologue(*p[9:]) if prologue is not None else None
    _check(load_library().xattn_bwd_noalloc(
        ctypes.byref(dims), *p[:9], ctypes.byref(pro) if pro is not None else None,
        _stream(stream)), "xattn_bwd_noalloc")


def make_decode_dims(xq, k_cache, num_heads, num_kv_heads, cache_len) -> DecodeDims:
    """xq: [B*H, q_len, hd]; k_cache: [B*Hkv, capacity, hd]."""
    bh, sq, hd = xq.shape
    if bh % num_heads:
        raise ValueError("xq.shape[0] must be batch * num_heads")
    B = bh // num_heads
    if k_cache.dim() != 3 or k_cache.shape[0] != B * num_kv_heads or k_cache.shape[2] != hd:
        raise ValueError(f"k_cache must be [batch * num_kv_heads, capacity, head_dim] = "
                         f"[{B * num_kv_heads}, capacity, {hd}], got {tuple(k_cache.shape)}")
    return DecodeDims(B, num_heads, num_kv_heads, hd, _io(xq, "xq"), sq, int(cache_len),
                      k_cache.shape[1])


def xattn_decode_workspace_bytes(dims: DecodeDims) -> int:
    return int(load_library().xattn_decode_workspace_bytes(ctypes.byref(dims)))


def _decode_ptrs(d, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, k_cache, v_cache, out, lse,
                 workspace, cache_lens=None):
    hd = d.head_dim
    nq = d.batch * d.num_heads * d.q_len * hd
    nk = d.batch * d.num_kv_heads * d.q_len * hd
    nc = d.batch * d.num_kv_heads * d.capacity * hd
    nt = d.capacity * (hd // 2)
    _io(xq, "xq")
    return _ptrs((xq, "xq", None, nq), (xk, "xk", xq.dtype, nk), (v, "v", xq.dtype, nk),
                 (gamma_q, "gamma_q", F32, hd), (gamma_k, "gamma_k", F32, hd),
                 (cos_tab, "cos_tab", F32, AtLeast(nt)), (sin_tab, "sin_tab", F32, AtLeast(nt)),
                 (k_cache, "k_cache", xq.dtype, nc), (v_cache, "v_cache", xq.dtype, nc),
                 (out, "out", xq.dtype, nq), (lse, "lse", F32, d.batch * d.num_heads * d.q_len),
                 (workspace, "workspace", None, None),
                 (cache_lens, "cache_lens", I32, d.batch))


def xattn_decode(dims: DecodeDims, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps,
                 k_cache, v_cache, out, lse, workspace, stream=None):
    p = _decode_ptrs(dims, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, k_cache, v_cache, out,
                     lse, workspace)
    _check(load_library().xattn_decode(
        ctypes.byref(dims), *p[:7], float(eps), *p[7:12], _bytes(workspace, "workspace"),
        _stream(stream)), "xattn_decode")


def xattn_decode_varlen(dims: DecodeDims, cache_lens, xq, xk, v, gamma_q, gamma_k, cos_tab,
                        sin_tab, eps, k_cache, v_cache, out, lse, workspace, stream=None):
    """cache_lens: int32 device tensor [batch], each sequence's cached rows (dims.cache_len
    must be their maximum)."""
    if cache_lens is None:
        raise ValueError("cache_lens must be an int32 device tensor")
    p = _decode_ptrs(dims, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, k_cache, v_cache, out,
                     lse, workspace, cache_lens)
    _check(load_library().xattn_decode_varlen(
        ctypes.byref(dims), p[12], *p[:7], float(eps), *p[7:12],
        _bytes(workspace, "workspace"), _stream(stream)), "xattn_decode_varlen")


# ----------------------------------------------------------------------------------------
# allocating helpers
# ----------------------------------------------------------------------------------------
def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def rope_cache(seq_len, head_dim, theta, device="cuda", stream=None):
    cos_tab = torch.empty(seq_len, head_dim // 2, dtype=torch.float32, device=device)
    sin_tab = torch.empty_like(cos_tab)
    xattn_rope_cache(cos_tab, sin_tab, seq_len, head_dim, theta, stream)
    return cos_tab, sin_tab


def qknorm_rope_fwd(x, gamma, cos_tab, sin_tab, eps, stream=None):
    rows, S, hd = x.shape
    y = torch.empty_like(x)
    rstd = torch.empty(rows * S, dtype=torch.float32, device=x.device)
    xattn_qknorm_rope_fwd(x, gamma, cos_tab, sin_tab, y, rstd, rows, S, hd, eps, stream)
    return y, rstd


def qknorm_rope_fwd_table(x, gamma, theta, eps, positions=None, stream=None):
    """QK-norm + RoPE of x with the RoPE table built in the same launch: (y, rstd, cos_tab,
    sin_tab); positions (int32 [S]) restart the angles per row as rope_cache_at does."""
    rows, S, hd = x.shape
    y = torch.empty_like(x)
    rstd = torch.empty(rows * S, dtype=torch.float32, device=x.device)
    cos_tab = torch.empty(S, hd // 2, dtype=torch.float32, device=x.device)
    sin_tab = torch.empty_like(cos_tab)
    xattn_qknorm_rope_fwd_table(x, gamma, positions, theta, cos_tab, sin_tab, y, rstd, rows, S,
                                hd, eps, stream)
    return y, rstd, cos_tab, sin_tab


def qknorm_rope_bwd(dy, x, gamma, rstd, cos_tab, sin_tab, stream=None, workspace=None):
    rows, S, hd = x.shape
    dx = torch.empty_like(x)
    dgamma = torch.empty(hd, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = _workspace(xattn_qknorm_rope_bwd_workspace_bytes(rows, S, hd), x.device)
    xattn_qknorm_rope_bwd(dy, x, gamma, rstd, cos_tab, sin_tab, dx, dgamma, workspace, rows, S,
                          hd, stream)
    return dx, dgamma


def segments(doc_lengths, device="cuda", stream=None):
    """Packed documents of the given lengths: (seg_lo, seg_hi, positions) int32 device
    tensors over the packed rows, built by xattn_segments from the document offsets."""
    offs = [0]
    for n in doc_lengths:
        offs.append(offs[-1] + int(n))
    cu = torch.tensor(offs, dtype=torch.int32, device=device)
    S = offs[-1]
    lo, hi, pos = (torch.empty(S, dtype=torch.int32, device=device) for _ in range(3))
    xattn_segments(cu, len(offs) - 1, S, lo, hi, pos, stream)
    return lo, hi, pos


def rope_cache_at(positions, head_dim, theta, stream=None):
    rows = positions.numel()
    cos_tab = torch.empty(rows, head_dim // 2, dtype=torch.float32, device=positions.device)
    sin_tab = torch.empty_like(cos_tab)
    xattn_rope_cache_at(cos_tab, sin_tab, positions, rows, head_dim, theta, stream)
    return cos_tab, sin_tab


def attn_fwd(q, k, v, num_heads, num_kv_heads, stream=None, segments=None):
    dims = make_dims(q, num_heads, num_kv_heads, segments)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0] * q.shape[1], dtype=torch.float32, device=q.device)
    xattn_fwd(dims, q, k, v, out, lse, stream)
    return out, lse


def attn_fwd_qnorm(xq, gamma_q, cos_tab, sin_tab, eps, k, v, num_heads, num_kv_heads,
                   stream=None, segments=None):
    """Forward with the Q-side QK-norm + RoPE fused; returns (out, lse, yq, rstd_q)."""
    dims = make_dims(xq, num_heads, num_kv_heads, segments)
    out, yq = torch.empty_like(xq), torch.empty_like(xq)
    lse = torch.empty(xq.shape[0] * xq.shape[1], dtype=torch.float32, device=xq.device)
    rstd_q = torch.empty_like(lse)
    xattn_fwd_qnorm(dims, xq, gamma_q, cos_tab, sin_tab, eps, yq, rstd_q, k, v, out, lse, stream)
    return out, lse, yq, rstd_q


def attn_bwd(q, k, v, out, lse, dout, num_heads, num_kv_heads, prologue=None, stream=None,
             workspace=None, segments=None):
    """Returns (dq, dk, dv); with a prologue dict (see xattn_bwd, without the dgamma
    entries) returns (dxq, dxk, dv, dgamma_q, dgamma_k)."""
    dims = make_dims(q, num_heads, num_kv_heads, segments)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pro = None
    if prologue is not None:
        hd = q.shape[-1]
        pro = dict(prologue)
        pro["dgamma_q"] = torch.empty(hd, dtype=torch.float32, device=q.device)
        pro["dgamma_k"] = torch.empty(hd, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = _workspace(xattn_bwd_workspace_bytes(dims, pro is not None), q.device)
    xattn_bwd(dims, q, k, v, out, lse, dout, dq, dk, dv, pro, workspace, stream)
    if pro is None:
        return dq, dk, dv
    return dq, dk, dv, pro["dgamma_q"], pro["dgamma_k"]


def decode(xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps, k_cache, v_cache, cache_len,
           num_heads, num_kv_heads, stream=None, workspace=None):
    """One KV-cache decode step: appends the new tokens' rotated keys and values to the
    caches (rows cache_len ..) and returns (out, lse) of the new queries.  cache_len: an int
    (every sequence), or an int32 device tensor [batch] of per-sequence lengths."""
    per_seq = isinstance(cache_len, torch.Tensor)
    dims = make_decode_dims(xq, k_cache, num_heads, num_kv_heads,
                            int(cache_len.max().item()) if per_seq else cache_len)
    out = torch.empty_like(xq)
    lse = torch.empty(xq.shape[0] * xq.shape[1], dtype=torch.float32, device=xq.device)
    if workspace is None:
        workspace = _workspace(xattn_decode_workspace_bytes(dims), xq.device)
    if per_seq:
        xattn_decode_varlen(dims, cache_len, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps,
                            k_cache, v_cache, out, lse, workspace, stream)
    else:
        xattn_decode(dims, xq, xk, v, gamma_q, gamma_k, cos_tab, sin_tab, eps, k_cache, v_cache,
                     out, lse, workspace, stream)
    return out, lse


class Projection:
    """The projections around attention for one shape: weights [d_in, d_out] (io dtype),
    optional fp32 biases; one preallocated workspace.  q/k/v/out tensors use the attention
    layouts ([B*H, S, hd], [B*Hkv, S, hd]); x, y are token rows [B*S, d]."""

    def __init__(self, batch, seq_len, num_heads, num_kv_heads, head_dim, wq, wk, wv, wo,
                 bq=None, bk=None, bv=None, bo=None):
        self.B, self.S, self.H, self.Hkv, self.hd = batch, seq_len, num_heads, num_kv_heads, head_dim
        if not isinstance(wq, torch.Tensor) or wq.dim() != 2:
            raise ValueError("wq must be a [model_dim, num_heads * head_dim] tensor")
        self.d = d = wq.shape[0]
        self.dt = wq.dtype
        self.nq, self.nk = nq, nk = num_heads * head_dim, num_kv_heads * head_dim
        self.M = batch * seq_len
        self.dims = Dims(batch, seq_len, num_heads, num_kv_heads, head_dim, _io(wq, "wq"))
        self._keep = (wq, wk, wv, wo, bq, bk, bv, bo)
        self.p = Proj(d, *_ptrs((wq, "wq", None, d * nq), (wk, "wk", self.dt, d * nk),
                                (wv, "wv", self.dt, d * nk), (wo, "wo", self.dt, nq * d),
                                (bq, "bq", F32, nq), (bk, "bk", F32, nk), (bv, "bv", F32, nk),
                                (bo, "bo", F32, d)))
        n = int(load_library().xattn_proj_workspace_bytes(ctypes.byref(self.dims), d))
        if n == 0:
            raise XattnError(1, "xattn_proj_workspace_bytes", xattn_last_error())
        self.ws = _workspace(n, wq.device)

    def _e(self, *shape, dtype=None):
        return torch.empty(shape, dtype=dtype or self.dt, device=self.ws.device)

    def _call(self, fn, specs, where, stream):
        p = _ptrs(*specs, (self.ws, "ws", None, None))
        _check(getattr(load_library(), fn)(ctypes.byref(self.dims), ctypes.byref(self.p), *p,
                                           _bytes(self.ws, "ws"), _stream(stream)), where)

    def qkv_fwd(self, x, stream=None):
        M, nq, nk, dt = self.M, self.nq, self.nk, self.dt
        xq, xk, v = self._e(self.B * self.H, self.S, self.hd), \
            self._e(self.B * self.Hkv, self.S, self.hd), self._e(self.B * self.Hkv, self.S, self.hd)
        self._call("xattn_qkv_proj_fwd", [(x, "x", dt, M * self.d), (xq, "xq", dt, M * nq),
                                          (xk, "xk", dt, M * nk), (v, "v", dt, M * nk)],
                   "xattn_qkv_proj_fwd", stream)
        return xq, xk, v

    def out_fwd(self, out, stream=None):
        y = self._e(self.M, self.d)
        self._call("xattn_out_proj_fwd", [(out, "out", self.dt, self.M * self.nq),
                                          (y, "y", self.dt, self.M * self.d)],
                   "xattn_out_proj_fwd", stream)
        return y

    def out_bwd(self, out, dy, with_bias=True, stream=None):
        M, nq, d, dt = self.M, self.nq, self.d, self.dt
        dout = self._e(self.B * self.H, self.S, self.hd)
        dwo = self._e(nq, d, dtype=F32)
        dbo = self._e(d, dtype=F32) if with_bias else None
        self._call("xattn_out_proj_bwd", [(out, "out", dt, M * nq), (dy, "dy", dt, M * d),
                                          (dout, "dout", dt, M * nq), (dwo, "dwo", F32, nq * d),
                                          (dbo, "dbo", F32, d)],
                   "xattn_out_proj_bwd", stream)
        return dout, dwo, dbo

    def qkv_bwd(self, x, dxq, dxk, dv, with_bias=True, stream=None):
        M, nq, nk, d, dt = self.M, self.nq, self.nk, self.d, self.dt
        dx = self._e(M, d)
        dw = [self._e(d, n, dtype=F32) for n in (nq, nk, nk)]
        db = [self._e(n, dtype=F32) if with_bias else None for n in (nq, nk, nk)]
        self._call("xattn_qkv_proj_bwd",
                   [(x, "x", dt, M * d), (dxq, "dxq", dt, M * nq), (dxk, "dxk", dt, M * nk),
                    (dv, "dv", dt, M * nk), (dx, "dx", dt, M * d),
                    (dw[0], "dwq", F32, d * nq), (dw[1], "dwk", F32, d * nk),
                    (dw[2], "dwv", F32, d * nk), (db[0], "dbq", F32, nq),
                    (db[1], "dbk", F32, nk), (db[2], "dbv", F32, nk)],
                   "xattn_qkv_proj_bwd", stream)
        return dx, dw, db
