"""Plain fp64 CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers.  The product library
never imports, links or runs anything here, and nothing here imports the
product package: the two share no code.  Inputs are the raw values the GPU
path receives (bf16 bit patterns as ``uint16``, fp32, int32); results are fp64.

The arithmetic lives in ``xo.c`` (plain C, one loop per term of each
definition; see the comments there for the passage each function follows).
This module only compiles it with gcc and marshals numpy arrays through ctypes.

Functions whose result has no independent pin would be marked "parity unpinned"
here; every function below is pinned by the CPU tests in ``tests/`` (brute-force
matrix algebra, exact rational arithmetic, closed forms and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "xo.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile xo.c into liboracle.so with gcc (fp64, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_c(_SRC, _LIB)
    return _LIB


def _bind(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.xo_version.restype = I
    lib.xo_gemm.argtypes = [P, P, P, I, I, I]
    lib.xo_gdn.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, P, P, P]
    lib.xo_rollback.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P, P]
    lib.xo_attn.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, P]
    lib.xo_attn_row.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, I, I, I, P]
    lib.xo_greedy.argtypes = [P, P, I, I, I, P, P]
    lib.xo_logprob.argtypes = [P, P, I, I, I, P]
    for f in ("xo_gemm", "xo_gdn", "xo_rollback", "xo_attn", "xo_attn_row", "xo_greedy", "xo_logprob"):
        getattr(lib, f).restype = None
    return lib


def compile_c(src: str, out: str) -> str:
    """gcc command used for the oracle (also used by the tests for planted-mistake copies)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build_sanitized(out_dir: str) -> str:
    """The oracle and its driver (sanitize_main.c: every function on edge shapes, with
    property checks) as one program built with AddressSanitizer and UndefinedBehavior-
    Sanitizer (a CPU check of the oracle's indexing; test infrastructure)."""
    out = os.path.join(out_dir, "xo_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", _SRC, os.path.join(_HERE, "sanitize_main.c"), "-o", out, "-lm"]
    subprocess.check_call(cmd)
    return out


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _bind(_LIB)
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def gemm(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] w[n][k] in fp64.  x: bf16 bits [M][K]; w: bf16 bits [N][K]."""
    x = _c(x, np.uint16); w = _c(w, np.uint16)
    M, K = x.shape
    N, K2 = w.shape
    assert K == K2
    y = np.empty((M, N), np.float64)
    _load().xo_gemm(_p(x), _p(w), _p(y), M, N, K)
    return y


def gdn(q, k, v, a, b, S0, *, want_all: bool = False):
    """Gated delta rule over T tokens for B requests.

    q, k: bf16 bits [B][T][Hk][dk]; v: bf16 bits [B][T][Hv][dv]; a, b: fp32 [B][T][Hv];
    S0: fp32 [B][Hv][dk][dv] (value index contiguous).
    Returns (o [B][T][Hv][dv], S_T [B][Hv][dk][dv], S_all [B][T+1][Hv][dk][dv] or None), fp64.
    """
    q = _c(q, np.uint16); k = _c(k, np.uint16); v = _c(v, np.uint16)
    a = _c(a, np.float32); b = _c(b, np.float32); S0 = _c(S0, np.float32)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and a.shape == (B, T, Hv) == b.shape
    assert S0.shape == (B, Hv, dk, dv)
    o = np.empty((B, T, Hv, dv), np.float64)
    ST = np.empty((B, Hv, dk, dv), np.float64)
    Sall = np.empty((B, T + 1, Hv, dk, dv), np.float64) if want_all else None
    _load().xo_gdn(_p(q), _p(k), _p(v), _p(a), _p(b), _p(S0), B, T, Hk, Hv, dk, dv,
                   _p(o), _p(Sall) if Sall is not None else None, _p(ST))
    return o, ST, Sall


def rollback(k, v, a, b, S0, kv_len, n_keep):
    """State after the first n_keep[b] rows (fp64) and kv_len + n_keep (int32)."""
    k = _c(k, np.uint16); v = _c(v, np.uint16)
    a = _c(a, np.float32); b = _c(b, np.float32); S0 = _c(S0, np.float32)
    kv_len = _c(kv_len, np.int32); n_keep = _c(n_keep, np.int32)
    B, T, Hk, dk = k.shape
    Hv, dv = v.shape[2], v.shape[3]
    Sn = np.empty((B, Hv, dk, dv), np.float64)
    kv_out = np.empty((B,), np.int32)
    _load().xo_rollback(_p(k), _p(v), _p(a), _p(b), _p(S0), _p(kv_len), _p(n_keep),
                        B, T, Hk, Hv, dk, dv, _p(Sn), _p(kv_out))
    return Sn, kv_out


def attn(q, k_new, v_new, k_cache, v_cache, kv_len, scale: float) -> np.ndarray:
    """Exact softmax attention, one decode row per verify row.  Returns fp64 [B][T][Hq][d]."""
    q = _c(q, np.uint16); k_new = _c(k_new, np.uint16); v_new = _c(v_new, np.uint16)
    k_cache = _c(k_cache, np.uint16); v_cache = _c(v_cache, np.uint16)
    kv_len = _c(kv_len, np.int32)
    B, T, Hq, d = q.shape
    Hkv = k_new.shape[2]
    Lmax = k_cache.shape[2]
    o = np.empty((B, T, Hq, d), np.float64)
    _load().xo_attn(_p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(kv_len),
                    B, T, Hq, Hkv, d, Lmax, float(scale), _p(o))
    return o


def attn_row(q, k_new, v_new, k_cache, v_cache, kv_len, scale: float, b: int, r: int, h: int):
    """One row (b, r, h) of :func:`attn`; fp64 [d]."""
    q = _c(q, np.uint16); k_new = _c(k_new, np.uint16); v_new = _c(v_new, np.uint16)
    k_cache = _c(k_cache, np.uint16); v_cache = _c(v_cache, np.uint16)
    kv_len = _c(kv_len, np.int32)
    B, T, Hq, d = q.shape
    Hkv = k_new.shape[2]
    Lmax = k_cache.shape[2]
    out = np.empty((d,), np.float64)
    _load().xo_attn_row(_p(q), _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(kv_len),
                        B, T, Hq, Hkv, d, Lmax, float(scale), int(b), int(r), int(h), _p(out))
    return out


def greedy(logits: np.ndarray, draft: np.ndarray):
    """Argmax ids (lowest index on ties) and accepted row counts.  logits fp64 [B][T][N]."""
    logits = _c(logits, np.float64); draft = _c(draft, np.int32)
    B, T, N = logits.shape
    ids = np.empty((B, T), np.int32)
    n_keep = np.empty((B,), np.int32)
    _load().xo_greedy(_p(logits), _p(draft), B, T, N, _p(ids), _p(n_keep))
    return ids, n_keep


def logprob(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """log softmax(logits[b][t])[ids[b][t]] in fp64.  logits fp64 [B][T][N]; ids int32 [B][T]."""
    logits = _c(logits, np.float64); ids = _c(ids, np.int32)
    B, T, N = logits.shape
    assert ids.shape == (B, T) and ids.min() >= 0 and ids.max() < N
    lp = np.empty((B, T), np.float64)
    _load().xo_logprob(_p(logits), _p(ids), B, T, N, _p(lp))
    return lp
