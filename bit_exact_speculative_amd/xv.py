"""Thin Python binding of libxv (ctypes).  Argument marshalling only.

Every function has the name of the C entry point it calls and takes device
tensors (PyTorch is used for device memory and streams, nothing else).  Sizes
are read from the tensor shapes, pointers from ``data_ptr()``, the stream from
``torch.cuda.current_stream()`` unless one is given.  A non-zero status from the
library raises :class:`XvError`.  There is no fallback of any kind: if libxv.so
is missing this module fails to import.

bf16 tensors may be ``torch.bfloat16`` or ``torch.int16`` / ``torch.uint16``
bit views; fp32 tensors are ``torch.float32``; lengths and ids ``torch.int32``.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxv.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "xv.h")

if not os.path.exists(LIB_PATH):
    raise ImportError("libxv.so is not built (%s); run __graft_entry__.build() first" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t

_lib.xv_abi_version.restype = _I
_lib.xv_abi_version.argtypes = []
_lib.xv_status_string.restype = ctypes.c_char_p
_lib.xv_status_string.argtypes = [_I]
# the argument lists below are those of this ABI version of include/xv.h
ABI_VERSION = 8
if _lib.xv_abi_version() != ABI_VERSION:
    raise ImportError("libxv.so has ABI version %d, this binding expects %d; rebuild it"
                      % (_lib.xv_abi_version(), ABI_VERSION))
_lib.xv_gemm_small_m.restype = _I
_lib.xv_gemm_small_m.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P]
_lib.xv_gemm_small_m_timed.restype = _I
_lib.xv_gemm_small_m_timed.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P]
_lib.xv_gemm_small_m_pair.restype = _I
_lib.xv_gemm_small_m_pair.argtypes = [_P, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P]
_lib.xv_gdn_verify.restype = _I
_lib.xv_gdn_verify.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
_lib.xv_attn_chunk_tokens.restype = _I
_lib.xv_attn_chunk_tokens.argtypes = []
_lib.xv_attn_workspace_bytes.restype = _S
_lib.xv_attn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.xv_attn_verify_rows.restype = _I
_lib.xv_attn_verify_rows.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _S,
                                     _I, _I, _I, _I, _I, _I, _F, _I, _P]
_lib.xv_attn_verify_rows_noalloc.restype = _I
_lib.xv_attn_verify_rows_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P,
                                             _I, _I, _I, _I, _I, _I, _F, _I, _P]
_lib.xv_stream_read.restype = _I
_lib.xv_stream_read.argtypes = [_P, _S, _P, _S, _P, _I, _P, _P, _P]
_lib.xv_rollback_to_prefix.restype = _I
_lib.xv_rollback_to_prefix.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]
_lib.xv_greedy_accept.restype = _I
_lib.xv_greedy_accept.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P]
_lib.xv_head_greedy_workspace_bytes.restype = _S
_lib.xv_head_greedy_workspace_bytes.argtypes = [_I, _I, _I]
_lib.xv_head_greedy_accept.restype = _I
_lib.xv_head_greedy_accept.argtypes = [_P] * 14 + [_S] + [_I] * 4 + [_P]
_lib.xv_gdn_prefill.restype = _I
_lib.xv_gdn_prefill.argtypes = [_P] * 9 + [_I] * 6 + [_P]
_lib.xv_attn_prefill.restype = _I
_lib.xv_attn_prefill.argtypes = [_P] * 8 + [_I] * 6 + [_F, _I, _P]
_lib.xv_gdn_attn_verify.restype = _I
_lib.xv_gdn_attn_verify.argtypes = ([_P] * 10 + [_I] + [_P] * 6 + [_I] * 4 + [_P] * 9 + [_S] +
                                    [_I] * 4 + [_F] + [_I, _I, _I, _P])
_lib.xv_gdn_verify_after.restype = _I
_lib.xv_gdn_verify_after.argtypes = [_P] * 10 + [_I] + [_P] * 6 + [_I] * 6 + [_P]
_lib.xv_embed_rows.restype = _I
_lib.xv_embed_rows.argtypes = [_P, _P, _I, _I, _I, _P, _P]
_lib.xv_split_projections.restype = _I
_lib.xv_split_projections.argtypes = [_P, _P, _I, _I, _I] + [_I] * 7 + [_P] * 8 + [_P]

XV_OK = 0
STATUS = {0: "XV_OK", -1: "XV_ERR_NULL", -2: "XV_ERR_SHAPE", -3: "XV_ERR_ALIGN",
          -4: "XV_ERR_WORKSPACE", -5: "XV_ERR_LAUNCH", -6: "XV_ERR_ALIAS"}


class XvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.xv_status_string(status).decode()
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), msg))


def lib():
    """The loaded ctypes library (for raw-pointer calls)."""
    return _lib


def exported_symbols_from_header(path: str = HEADER_PATH):
    """Names of every function the C header declares."""
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xv_[a-z0-9_]+)\s*\(", src)))


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libxv must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != XV_OK:
        raise XvError(fn, status)


def xv_abi_version() -> int:
    return _lib.xv_abi_version()


def xv_attn_chunk_tokens() -> int:
    return _lib.xv_attn_chunk_tokens()


def xv_attn_workspace_bytes(B: int, T: int, Hq: int, d: int, Lmax: int) -> int:
    return int(_lib.xv_attn_workspace_bytes(B, T, Hq, d, Lmax))


ATTN_COUNTER_BYTES = 4096    # the attention workspace's leading arrival counters


def xv_attn_workspace(B: int, T: int, Hq: int, d: int, Lmax: int, device="cuda", fill=None):
    """A float32 workspace for the attention calls: its arrival counters (the first 4096
    bytes) zero, the partials after them zero or `fill`."""
    import torch
    n = (max(xv_attn_workspace_bytes(B, T, Hq, d, Lmax), ATTN_COUNTER_BYTES) + 15) // 16 * 4
    ws = torch.zeros((n,), dtype=torch.float32, device=device)
    if fill is not None:
        ws[ATTN_COUNTER_BYTES // 4:].fill_(fill)
    return ws


def xv_gemm_small_m(x, w, y, y32=None, stream=None):
    """y[M][N] (bf16) = x[M][K] @ w[N][K]^T; y32 optional fp32 copy before rounding."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N) or (y32 is not None and tuple(y32.shape) != (M, N)):
        raise ValueError("xv_gemm_small_m: shape mismatch")
    _check("xv_gemm_small_m", _lib.xv_gemm_small_m(_ptr(x), _ptr(w), _ptr(y), _ptr(y32),
                                                  M, N, K, _stream(stream)))


def _event(e):
    """Raw hipEvent_t of a torch.cuda.Event (created on first use), or None."""
    if e is None:
        return None
    if not e.cuda_event:
        e.record()                     # torch creates the event lazily
    return e.cuda_event


def xv_gemm_small_m_timed(x, w, y, y32=None, start=None, stop=None, stream=None):
    """xv_gemm_small_m with torch.cuda.Event start / stop recorded by the launch itself."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(y.shape) != (M, N) or (y32 is not None and tuple(y32.shape) != (M, N)):
        raise ValueError("xv_gemm_small_m_timed: shape mismatch")
    _check("xv_gemm_small_m_timed", _lib.xv_gemm_small_m_timed(_ptr(x), _ptr(w), _ptr(y), _ptr(y32),
                                                              M, N, K, _stream(stream),
                                                              _event(start), _event(stop)))


def xv_gemm_small_m_pair(x0, w0, y0, y32_0, x1, w1, y1, y32_1, start=None, stop=None, stream=None):
    """y0 = x0 @ w0^T and y1 = x1 @ w1^T (same M and K) in one launch; optional fp32 copies
    and torch.cuda.Event start / stop recorded by the launch itself."""
    M, K = x0.shape
    N0, N1 = w0.shape[0], w1.shape[0]
    if tuple(x1.shape) != (M, K) or w0.shape[1] != K or w1.shape[1] != K or \
            tuple(y0.shape) != (M, N0) or tuple(y1.shape) != (M, N1) or \
            (y32_0 is not None and tuple(y32_0.shape) != (M, N0)) or \
            (y32_1 is not None and tuple(y32_1.shape) != (M, N1)):
        raise ValueError("xv_gemm_small_m_pair: shape mismatch")
    _check("xv_gemm_small_m_pair", _lib.xv_gemm_small_m_pair(
        _ptr(x0), _ptr(w0), _ptr(y0), _ptr(y32_0), N0, _ptr(x1), _ptr(w1), _ptr(y1), _ptr(y32_1), N1,
        M, K, _stream(stream), _event(start), _event(stop)))


def xv_gdn_verify(q, k, v, a, b, state_in, state_out, o, o32=None, stream=None):
    """Gated delta rule over T rows: shapes q,k [B][T][Hk][dk], v [B][T][Hv][dv], ..."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if tuple(k.shape) != (B, T, Hk, dk) or tuple(v.shape[:2]) != (B, T) or \
            tuple(a.shape) != (B, T, Hv) or tuple(b.shape) != (B, T, Hv) or \
            tuple(state_in.shape) != (B, Hv, dk, dv) or tuple(state_out.shape) != (B, Hv, dk, dv) or \
            tuple(o.shape) != (B, T, Hv, dv) or (o32 is not None and tuple(o32.shape) != (B, T, Hv, dv)):
        raise ValueError("xv_gdn_verify: shape mismatch")
    _check("xv_gdn_verify", _lib.xv_gdn_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                              _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(o32),
                                              B, T, Hk, Hv, dk, dv, _stream(stream)))


def xv_gdn_verify_after(q, k, v, a, b, k_prev, v_prev, a_prev, b_prev, n_keep_prev,
                        state_prev_in, state_prev_out, state_kept, state_out, o, o32=None, stream=None):
    """The kept rows of the previous verify (k_prev .. b_prev, n_keep_prev) replayed from
    state_prev_in (or state_prev_out when all were kept) into state_kept, then a verify of
    this call's rows from it into state_out; as xv_rollback_to_prefix + xv_gdn_verify."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    Tp = k_prev.shape[1]
    st = (B, Hv, dk, dv)
    if tuple(k.shape) != (B, T, Hk, dk) or tuple(v.shape[:2]) != (B, T) or \
            tuple(a.shape) != (B, T, Hv) or tuple(b.shape) != (B, T, Hv) or \
            tuple(k_prev.shape) != (B, Tp, Hk, dk) or tuple(v_prev.shape) != (B, Tp, Hv, dv) or \
            tuple(a_prev.shape) != (B, Tp, Hv) or tuple(b_prev.shape) != (B, Tp, Hv) or \
            tuple(n_keep_prev.shape) != (B,) or \
            any(tuple(s.shape) != st for s in (state_prev_in, state_prev_out, state_kept, state_out)) or \
            tuple(o.shape) != (B, T, Hv, dv) or (o32 is not None and tuple(o32.shape) != (B, T, Hv, dv)):
        raise ValueError("xv_gdn_verify_after: shape mismatch")
    _check("xv_gdn_verify_after", _lib.xv_gdn_verify_after(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(k_prev), _ptr(v_prev), _ptr(a_prev),
        _ptr(b_prev), _ptr(n_keep_prev), Tp, _ptr(state_prev_in), _ptr(state_prev_out),
        _ptr(state_kept), _ptr(state_out), _ptr(o), _ptr(o32), B, T, Hk, Hv, dk, dv, _stream(stream)))


def xv_gdn_attn_verify(q, k, v, a, b, state_in, state_out, o, q_attn, k_new, v_new, k_cache, v_cache,
                       kv_len, o_attn, workspace, scale=None, o32=None, o_attn32=None, prev=None,
                       len_bound=0, stream=None):
    """GDN verify and attention verify rows in one call (one launch when they fit the chip).
    prev: None (as xv_gdn_verify), or (k_prev, v_prev, a_prev, b_prev, n_keep_prev,
    state_prev_out, state_kept) for xv_gdn_verify_after from state_in; then as
    xv_attn_verify_rows (len_bound: 0, or an upper bound on kv_len[b] + T)."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    Hq, d = q_attn.shape[2], q_attn.shape[3]
    Hkv, Lmax = k_new.shape[2], k_cache.shape[2]
    st = (B, Hv, dk, dv)
    bad = tuple(k.shape) != (B, T, Hk, dk) or tuple(v.shape[:2]) != (B, T) or \
        tuple(a.shape) != (B, T, Hv) or tuple(b.shape) != (B, T, Hv) or \
        tuple(state_in.shape) != st or tuple(state_out.shape) != st or tuple(o.shape) != (B, T, Hv, dv) or \
        (o32 is not None and tuple(o32.shape) != (B, T, Hv, dv)) or \
        tuple(q_attn.shape[:2]) != (B, T) or tuple(k_new.shape) != (B, T, Hkv, d) or \
        tuple(v_new.shape) != (B, T, Hkv, d) or tuple(k_cache.shape) != (B, Hkv, Lmax, d) or \
        tuple(v_cache.shape) != (B, Hkv, Lmax, d) or tuple(kv_len.shape) != (B,) or \
        tuple(o_attn.shape) != (B, T, Hq, d) or (o_attn32 is not None and tuple(o_attn32.shape) != (B, T, Hq, d))
    Tp = 0
    if prev is not None:
        kp, vp, ap, bp, nk, sp, sk = prev
        Tp = kp.shape[1]
        bad = bad or tuple(kp.shape) != (B, Tp, Hk, dk) or tuple(vp.shape) != (B, Tp, Hv, dv) or \
            tuple(ap.shape) != (B, Tp, Hv) or tuple(bp.shape) != (B, Tp, Hv) or tuple(nk.shape) != (B,) or \
            tuple(sp.shape) != st or tuple(sk.shape) != st
    else:
        kp = vp = ap = bp = nk = sp = sk = None
    if bad:
        raise ValueError("xv_gdn_attn_verify: shape mismatch")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    wbytes = workspace.numel() * workspace.element_size()
    _check("xv_gdn_attn_verify", _lib.xv_gdn_attn_verify(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(kp), _ptr(vp), _ptr(ap), _ptr(bp), _ptr(nk), Tp,
        _ptr(state_in), _ptr(sp), _ptr(sk), _ptr(state_out), _ptr(o), _ptr(o32), Hk, Hv, dk, dv,
        _ptr(q_attn), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
        _ptr(o_attn), _ptr(o_attn32), _ptr(workspace), wbytes, Hq, Hkv, d, Lmax, float(scale),
        B, T, int(len_bound), _stream(stream)))


def xv_gdn_prefill(q, k, v, a, b, state_in, state_out, o, o32=None, stream=None):
    """GDN over a whole prompt (any T), every row kept; shapes as xv_gdn_verify."""
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    if tuple(k.shape) != (B, T, Hk, dk) or tuple(v.shape[:2]) != (B, T) or \
            tuple(a.shape) != (B, T, Hv) or tuple(b.shape) != (B, T, Hv) or \
            tuple(state_in.shape) != (B, Hv, dk, dv) or tuple(state_out.shape) != (B, Hv, dk, dv) or \
            tuple(o.shape) != (B, T, Hv, dv) or (o32 is not None and tuple(o32.shape) != (B, T, Hv, dv)):
        raise ValueError("xv_gdn_prefill: shape mismatch")
    _check("xv_gdn_prefill", _lib.xv_gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                                _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(o32),
                                                B, T, Hk, Hv, dk, dv, _stream(stream)))


def xv_attn_prefill(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32=None, scale=None, advance=False,
                    stream=None):
    """P prompt rows at once: appends k_new / v_new at kv_len and forms every row's attention
    with the decode row's arithmetic (advance: then kv_len += P).  q [B][P][Hq][d]; k_new,
    v_new [B][P][Hkv][d]."""
    B, P, Hq, d = q.shape
    Hkv = k_new.shape[2]
    Lmax = k_cache.shape[2]
    if tuple(k_new.shape) != (B, P, Hkv, d) or tuple(v_new.shape) != (B, P, Hkv, d) or \
            tuple(k_cache.shape) != (B, Hkv, Lmax, d) or tuple(v_cache.shape) != (B, Hkv, Lmax, d) or \
            tuple(kv_len.shape) != (B,) or tuple(o.shape) != (B, P, Hq, d) or \
            (o32 is not None and tuple(o32.shape) != (B, P, Hq, d)):
        raise ValueError("xv_attn_prefill: shape mismatch")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    _check("xv_attn_prefill", _lib.xv_attn_prefill(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(o), _ptr(o32),
        B, P, Hq, Hkv, d, Lmax, float(scale), 1 if advance else 0, _stream(stream)))


def xv_attn_verify_rows(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32=None, workspace=None,
                        scale=None, len_bound=0, stream=None):
    """Attention rows + KV append.  q [B][T][Hq][d]; caches [B][Hkv][Lmax][d]; kv_len int32 [B];
    len_bound: 0, or an upper bound on kv_len[b] + T that sizes the launch (the same bits)."""
    B, T, Hq, d = q.shape
    Hkv = k_new.shape[2]
    Lmax = k_cache.shape[2]
    if tuple(k_new.shape) != (B, T, Hkv, d) or tuple(v_new.shape) != (B, T, Hkv, d) or \
            tuple(k_cache.shape) != (B, Hkv, Lmax, d) or tuple(v_cache.shape) != (B, Hkv, Lmax, d) or \
            tuple(kv_len.shape) != (B,) or tuple(o.shape) != (B, T, Hq, d) or \
            (o32 is not None and tuple(o32.shape) != (B, T, Hq, d)):
        raise ValueError("xv_attn_verify_rows: shape mismatch")
    if workspace is None:
        raise ValueError("xv_attn_verify_rows: a workspace tensor is required")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    wbytes = workspace.numel() * workspace.element_size()
    _check("xv_attn_verify_rows", _lib.xv_attn_verify_rows(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
        _ptr(o), _ptr(o32), _ptr(workspace), wbytes, B, T, Hq, Hkv, d, Lmax, float(scale),
        int(len_bound), _stream(stream)))


def xv_attn_verify_rows_noalloc(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32=None, scale=None,
                                len_bound=0, stream=None):
    """xv_attn_verify_rows with the library's own device buffer for the partials (no workspace)."""
    B, T, Hq, d = q.shape
    Hkv = k_new.shape[2]
    Lmax = k_cache.shape[2]
    if tuple(k_new.shape) != (B, T, Hkv, d) or tuple(v_new.shape) != (B, T, Hkv, d) or \
            tuple(k_cache.shape) != (B, Hkv, Lmax, d) or tuple(v_cache.shape) != (B, Hkv, Lmax, d) or \
            tuple(kv_len.shape) != (B,) or tuple(o.shape) != (B, T, Hq, d) or \
            (o32 is not None and tuple(o32.shape) != (B, T, Hq, d)):
        raise ValueError("xv_attn_verify_rows_noalloc: shape mismatch")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    _check("xv_attn_verify_rows_noalloc", _lib.xv_attn_verify_rows_noalloc(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_len),
        _ptr(o), _ptr(o32), B, T, Hq, Hkv, d, Lmax, float(scale), int(len_bound), _stream(stream)))


def xv_stream_read(src0, src1, sink, start_event=None, stop_event=None, stream=None):
    """Read src0 and src1 once (measurement helper); sink: int32/uint32 [workgroups]."""
    b0 = src0.numel() * src0.element_size()
    b1 = 0 if src1 is None else src1.numel() * src1.element_size()
    _check("xv_stream_read", _lib.xv_stream_read(
        _ptr(src0), b0, _ptr(src1), b1, _ptr(sink), sink.numel(), _stream(stream),
        _event(start_event), _event(stop_event)))


def xv_rollback_to_prefix(k, v, a, b, state_in, state_out, kv_len, n_keep, stream=None):
    """Keep n_keep[b] verify rows: state_out <- S_n, kv_len += n."""
    B, T, Hk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    if tuple(state_in.shape) != (B, Hv, dk, dv) or tuple(state_out.shape) != (B, Hv, dk, dv) or \
            tuple(kv_len.shape) != (B,) or tuple(n_keep.shape) != (B,):
        raise ValueError("xv_rollback_to_prefix: shape mismatch")
    _check("xv_rollback_to_prefix", _lib.xv_rollback_to_prefix(
        _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(state_in), _ptr(state_out), _ptr(kv_len),
        _ptr(n_keep), B, T, Hk, Hv, dk, dv, _stream(stream)))


def xv_greedy_accept(logits_a, logits_b, draft, ids, n_keep, logprob=None, stream=None, kv_len=None):
    """ids = argmax(logits_a + logits_b) per row (lowest index on ties); n_keep per request;
    logprob (optional fp32 [B][T]) = log-softmax of each row at its id; kv_len (optional
    int32 [B]) += n_keep."""
    B, T, N = logits_a.shape
    if (logits_b is not None and tuple(logits_b.shape) != (B, T, N)) or tuple(draft.shape) != (B, T) \
            or tuple(ids.shape) != (B, T) or tuple(n_keep.shape) != (B,) or \
            (logprob is not None and tuple(logprob.shape) != (B, T)) or \
            (kv_len is not None and tuple(kv_len.shape) != (B,)):
        raise ValueError("xv_greedy_accept: shape mismatch")
    _check("xv_greedy_accept", _lib.xv_greedy_accept(_ptr(logits_a), _ptr(logits_b), _ptr(draft),
                                                    B, T, N, _ptr(ids), _ptr(n_keep), _ptr(logprob),
                                                    _ptr(kv_len), _stream(stream)))


def xv_head_greedy_workspace_bytes(B: int, T: int, N: int) -> int:
    return int(_lib.xv_head_greedy_workspace_bytes(B, T, N))


def xv_head_greedy_accept(x_a, w_a, y_a, logits_a, x_b, w_b, y_b, logits_b, draft, ids, n_keep,
                          workspace, logprob=None, kv_len=None, stream=None):
    """The head pair (x_a @ w_a^T, x_b @ w_b^T over M = B*T rows) and greedy acceptance on
    logits_a + logits_b in one call: the outputs of xv_gemm_small_m_pair followed by
    xv_greedy_accept.  workspace: a uint8 device tensor of xv_head_greedy_workspace_bytes
    bytes, zero before its first use (each call leaves it ready for the next)."""
    B, T = draft.shape
    M, K = x_a.shape
    N = w_a.shape[0]
    if M != B * T or tuple(x_b.shape) != (M, K) or tuple(w_a.shape) != (N, K) or \
            tuple(w_b.shape) != (N, K) or tuple(y_a.shape) != (M, N) or tuple(y_b.shape) != (M, N) or \
            tuple(logits_a.shape) != (M, N) or tuple(logits_b.shape) != (M, N) or \
            tuple(ids.shape) != (B, T) or tuple(n_keep.shape) != (B,) or \
            (logprob is not None and tuple(logprob.shape) != (B, T)) or \
            (kv_len is not None and tuple(kv_len.shape) != (B,)):
        raise ValueError("xv_head_greedy_accept: shape mismatch")
    _check("xv_head_greedy_accept", _lib.xv_head_greedy_accept(
        _ptr(x_a), _ptr(w_a), _ptr(y_a), _ptr(logits_a), _ptr(x_b), _ptr(w_b), _ptr(y_b), _ptr(logits_b),
        _ptr(draft), _ptr(ids), _ptr(n_keep), _ptr(logprob), _ptr(kv_len), _ptr(workspace),
        workspace.numel() * workspace.element_size(), B, T, N, K, _stream(stream)))


def xv_embed_rows(table, tokens, x, stream=None):
    """x[m] = table[tokens[m]] (bf16 rows).  table [V][H]; tokens int32 [M] (any shape of M ids)."""
    V, H = table.shape
    M = tokens.numel()
    if tuple(x.shape) != (M, H):
        raise ValueError("xv_embed_rows: shape mismatch")
    _check("xv_embed_rows", _lib.xv_embed_rows(_ptr(table), _ptr(tokens), M, V, H, _ptr(x),
                                              _stream(stream)))


def xv_split_projections(y1, y2, q, k, v, a, b, q_attn, k_new, v_new, stream=None):
    """Per-head operands from the projection rows y1 [M][N1], y2 [M][N2]; outputs are
    [M][heads][dim] (or the same memory as [B][T][heads][dim]); a, b fp32 [M][Hv]."""
    M, N1 = y1.shape
    N2 = y2.shape[1]
    Hk, dk = q.shape[-2], q.shape[-1]
    Hv, dv = v.shape[-2], v.shape[-1]
    Hq, d = q_attn.shape[-2], q_attn.shape[-1]
    Hkv = k_new.shape[-2]
    if y2.shape[0] != M or q.numel() != M * Hk * dk or k.numel() != M * Hk * dk or \
            v.numel() != M * Hv * dv or a.numel() != M * Hv or b.numel() != M * Hv or \
            q_attn.numel() != M * Hq * d or k_new.numel() != M * Hkv * d or v_new.numel() != M * Hkv * d:
        raise ValueError("xv_split_projections: shape mismatch")
    _check("xv_split_projections", _lib.xv_split_projections(
        _ptr(y1), _ptr(y2), M, N1, N2, Hk, Hv, dk, dv, Hq, Hkv, d,
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(q_attn), _ptr(k_new), _ptr(v_new),
        _stream(stream)))
