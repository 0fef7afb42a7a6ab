"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed: no call here reaches a
kernel launch or any other HIP runtime call)."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_exact_speculative_amd", "libxv.so")


@pytest.fixture(scope="module")
def xv():
    if not os.path.exists(LIB):
        from bit_exact_speculative_amd import build
        build.build()
    import bit_exact_speculative_amd.xv as m
    return m


def test_every_header_symbol_is_exported(xv):
    names = xv.exported_symbols_from_header()
    assert set(names) >= {"xv_gemm_small_m", "xv_gdn_verify", "xv_attn_verify_rows",
                          "xv_rollback_to_prefix", "xv_attn_workspace_bytes",
                          "xv_attn_chunk_tokens", "xv_abi_version", "xv_status_string",
                          "xv_greedy_accept", "xv_embed_rows", "xv_split_projections",
                          "xv_gemm_small_m_pair", "xv_gdn_verify_after", "xv_gdn_attn_verify",
                          "xv_attn_prefill", "xv_gdn_prefill", "xv_attn_verify_rows_noalloc",
                          "xv_head_greedy_accept", "xv_head_greedy_workspace_bytes"}
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_version_and_constants(xv):
    assert xv.xv_abi_version() == xv.ABI_VERSION == 8
    assert xv.xv_attn_chunk_tokens() == 256
    lib = xv.lib()
    assert lib.xv_status_string(0) == b"ok"
    assert lib.xv_status_string(-4) == b"workspace too small"
    # workspace: 4096 bytes of arrival counters, then B*T*Hq*nchunks*(d+2) fp32 partials
    assert xv.xv_attn_workspace_bytes(1, 9, 24, 256, 649) == 4096 + 1 * 9 * 24 * 3 * 258 * 4
    assert xv.xv_attn_workspace_bytes(8, 9, 24, 256, 256) == 4096 + 8 * 9 * 24 * 1 * 258 * 4
    assert xv.xv_attn_workspace_bytes(0, 9, 24, 256, 256) == 0


A = 0x10000            # a fake, 16-byte aligned device address (never dereferenced)
MIS = 0x10004          # 4-byte aligned, not 16-byte aligned
ODD = 0x10001          # not even 2-byte aligned


def test_gemm_argument_errors(xv):
    f = xv.lib().xv_gemm_small_m
    assert f(A, A, A, None, 0, 16, 32, None) == 0              # empty: ok, no launch
    assert f(None, A, A, None, 9, 16, 32, None) == -1
    assert f(A, A, None, None, 9, 16, 32, None) == -1
    assert f(A, A, A, None, 9, 15, 32, None) == -2             # N % 16
    assert f(A, A, A, None, 9, 16, 48, None) == -2             # K % 32
    assert f(A, A, A, None, -1, 16, 32, None) == -2
    assert f(A, A, A, None, 9, 0, 32, None) == -2
    assert f(A, MIS, A, None, 9, 16, 32, None) == -3
    assert f(A, A, ODD, None, 9, 16, 32, None) == -3
    assert f(A, A, A, A + 2, 9, 16, 32, None) == -3


def test_gemm_pair_argument_errors(xv):
    f = xv.lib().xv_gemm_small_m_pair

    def call(x0=A, w0=A, y0=A, N0=64, x1=A, w1=A, y1=A, N1=32, M=9, K=5120, y32_0=None, y32_1=None):
        return f(x0, w0, y0, y32_0, N0, x1, w1, y1, y32_1, N1, M, K, None, None, None)

    assert call(M=0) == 0
    assert call(N0=8) == -2 and call(N1=40) == -2 and call(K=48) == -2 and call(M=-1) == -2
    assert call(x1=None) == -1 and call(w0=None) == -1 and call(y1=None) == -1
    assert call(w1=MIS) == -3 and call(x0=MIS) == -3 and call(y0=ODD) == -3 and call(y32_1=A + 2) == -3


def test_gdn_argument_errors(xv):
    f = xv.lib().xv_gdn_verify
    ok = dict(B=1, T=9, Hk=16, Hv=48, dk=128, dv=128)

    def call(q=A, k=A, v=A, a=A, b=A, si=A, so=A + 0x100000, o=A, o32=None, **kw):
        s = dict(ok); s.update(kw)
        return f(q, k, v, a, b, si, so, o, o32, s["B"], s["T"], s["Hk"], s["Hv"], s["dk"], s["dv"], None)

    assert call(B=0) == 0
    assert call(T=0) == -2 and call(T=17) == -2
    assert call(Hv=47) == -2 and call(dk=96) == -2 and call(dv=16) == -2 and call(dv=160) == -2
    assert call(q=None) == -1 and call(si=None) == -1 and call(o=None) == -1
    assert call(k=MIS) == -3 and call(q=MIS) == -3 and call(o32=A + 2) == -3 and call(a=ODD) == -3
    assert call(si=MIS) == -3 and call(so=A + 0x100004) == -3   # states are read 16 bytes at a time
    assert call(so=A) == -6                                     # state_out aliases state_in
    r = xv.lib().xv_rollback_to_prefix
    assert r(A, A, A, A, A, A + 0x1000, None, A, 1, 9, 16, 48, 128, 128, None) == -1
    assert r(A, A, A, A, A, A, A, A, 1, 9, 16, 48, 128, 128, None) == -6
    assert r(A, A, A, A, A, A + 0x1000, A, A, 0, 9, 16, 48, 128, 128, None) == 0


def test_gdn_prefill_argument_errors(xv):
    f = xv.lib().xv_gdn_prefill

    def call(q=A, si=A, so=A + 0x100000, o=A, T=9000, B=1, dk=128, dv=128):
        return f(q, A, A, A, A, si, so, o, None, B, T, 16, 48, dk, dv, None)

    assert call(B=0) == 0
    assert call(T=0) == -2 and call(dk=96) == -2 and call(dv=16) == -2
    assert call(q=None) == -1 and call(o=None) == -1
    assert call(q=MIS) == -3 and call(so=A) == -6


def test_gdn_verify_after_argument_errors(xv):
    f = xv.lib().xv_gdn_verify_after
    ok = dict(Tp=9, B=1, T=9, Hk=16, Hv=48, dk=128, dv=128)
    S = [A + 0x100000 * i for i in range(4)]     # four distinct 16-byte aligned states

    def call(q=A, kp=A, vp=A, nk=A, si=S[0], sp=S[1], sk=S[2], so=S[3], o=A, o32=None, **kw):
        s = dict(ok); s.update(kw)
        return f(q, A, A, A, A, kp, vp, A, A, nk, s["Tp"], si, sp, sk, so, o, o32,
                 s["B"], s["T"], s["Hk"], s["Hv"], s["dk"], s["dv"], None)

    assert call(B=0) == 0
    assert call(Tp=0) == -2 and call(Tp=17) == -2 and call(T=17) == -2 and call(dk=96) == -2
    assert call(kp=None) == -1 and call(nk=None) == -1 and call(sk=None) == -1 and call(sp=None) == -1
    assert call(q=None) == -1 and call(o=None) == -1
    assert call(kp=MIS) == -3 and call(vp=ODD) == -3 and call(sk=S[2] + 4) == -3 and call(nk=A + 2) == -3
    for bad in (dict(so=S[0]), dict(so=S[1]), dict(sk=S[0]), dict(sk=S[1]), dict(sk=S[3])):
        assert call(**bad) == -6, bad


def test_gdn_attn_argument_errors(xv):
    """The combined call reports the first failing check of the two calls it stands for."""
    f = xv.lib().xv_gdn_attn_verify
    need = xv.xv_attn_workspace_bytes(1, 9, 24, 256, 649)
    S = [A + 0x100000 * i for i in range(4)]

    def call(nk=None, kp=None, si=S[0], sp=None, sk=None, so=S[1], T=9, dk=128, d=256, B=1, wsb=need,
             q=A, qa=A, kvl=A, Tp=0, lb=0):
        return f(q, A, A, A, A, kp, kp, kp, kp, nk, Tp, si, sp, sk, so, A, None, 16, 48, dk, 128,
                 qa, A, A, A, A, kvl, A, None, A, wsb, 24, 4, d, 649, 0.0625, B, T, lb, None)

    assert call(B=0) == 0
    assert call(T=17) == -2 and call(dk=96) == -2 and call(d=96) == -2
    assert call(lb=8) == -2 and call(lb=-1) == -2                # a length bound below T
    assert call(q=None) == -1 and call(qa=None) == -1 and call(kvl=None) == -1
    assert call(so=S[0]) == -6                                  # GDN state_out aliases state_in
    assert call(wsb=need - 4) == -4
    assert call(nk=A, Tp=9) == -1                               # after a verify: its rows are needed
    assert call(nk=A, Tp=0, kp=A, sp=S[2], sk=S[3]) == -2       # T_prev
    assert call(nk=A, Tp=9, kp=A, sp=S[2], sk=S[0]) == -6       # state_kept aliases state_in


def test_attn_prefill_argument_errors(xv):
    f = xv.lib().xv_attn_prefill

    def call(q=A, o=A, kvl=A, B=1, P=100, Hq=24, Hkv=4, d=256, Lmax=1000, scale=0.0625):
        return f(q, A, A, A, A, kvl, o, None, B, P, Hq, Hkv, d, Lmax, scale, 0, None)

    assert call(B=0) == 0
    assert call(P=0) == -2 and call(Hq=25) == -2 and call(d=96) == -2 and call(Lmax=99) == -2
    assert call(scale=float("nan")) == -2
    assert call(q=None) == -1 and call(kvl=None) == -1 and call(o=None) == -1
    assert call(q=MIS) == -3 and call(o=ODD) == -3


def test_attn_argument_errors(xv):
    f = xv.lib().xv_attn_verify_rows
    need = xv.xv_attn_workspace_bytes(1, 9, 24, 256, 649)

    def call(ws=A, wsb=need, B=1, T=9, Hq=24, Hkv=4, d=256, Lmax=649, q=A, kvl=A, scale=0.0625, lb=0):
        return f(q, A, A, A, A, kvl, A, None, ws, wsb, B, T, Hq, Hkv, d, Lmax, scale, lb, None)

    assert call(B=0) == 0 and call(B=0, lb=649) == 0
    assert call(T=17) == -2 and call(Hq=25) == -2 and call(d=96) == -2 and call(Lmax=8) == -2
    assert call(lb=8) == -2 and call(lb=-5) == -2                # a length bound below T
    assert call(B=1 << 13, T=16, Hq=64, Hkv=64, Lmax=1 << 20) == -2   # grid past 2^30 workgroups
    assert call(scale=float("nan")) == -2
    assert call(q=None) == -1 and call(kvl=None) == -1 and call(ws=None) == -1
    assert call(q=MIS) == -3
    assert call(wsb=need - 4) == -4


def test_attn_noalloc_argument_errors(xv):
    """Every failing check returns before any device call (only error cases are called: a
    valid call would launch on the fake pointers)."""
    f = xv.lib().xv_attn_verify_rows_noalloc
    limit = 32 << 20

    def call(B=1, T=9, Hq=24, Hkv=4, d=256, Lmax=649, q=A, kvl=A, o=A, scale=0.0625, lb=0):
        return f(q, A, A, A, A, kvl, o, None, B, T, Hq, Hkv, d, Lmax, scale, lb, None)

    assert call(B=0) == 0
    assert call(T=17) == -2 and call(Hq=25) == -2 and call(d=96) == -2 and call(Lmax=8) == -2
    assert call(scale=float("nan")) == -2
    assert call(q=None) == -1 and call(kvl=None) == -1 and call(o=None) == -1
    assert call(q=MIS) == -3
    # the library's array holds 32 MiB: the long context (127,744 positions) does not fit
    assert xv.xv_attn_workspace_bytes(1, 9, 24, 256, 127744) > limit
    assert call(Lmax=127744) == -4
    big_b = limit // xv.xv_attn_workspace_bytes(1, 9, 24, 256, 2560) + 1
    assert call(B=big_b, Lmax=2560) == -4


def test_stream_read_argument_errors(xv):
    f = xv.lib().xv_stream_read
    assert f(A, 0, A, 0, A, 1, None, None, None) == 0                # nothing to read: no launch
    assert f(A, 1024, A, 1024, A, 0, None, None, None) == -2          # no workgroups
    assert f(A, 1000, A, 1024, A, 8, None, None, None) == -2          # not whole 16-byte words
    assert f(None, 1024, A, 1024, A, 8, None, None, None) == -1
    assert f(A, 1024, A, 1024, None, 8, None, None, None) == -1
    assert f(MIS, 1024, A, 1024, A, 8, None, None, None) == -3


def test_greedy_argument_errors(xv):
    f = xv.lib().xv_greedy_accept
    assert f(A, None, A, 0, 9, 4096, A, A, None, None, None) == 0
    assert f(A, None, A, 1, 0, 4096, A, A, None, None, None) == -2
    assert f(A, None, A, 1, 9, 0, A, A, None, None, None) == -2
    assert f(None, None, A, 1, 9, 4096, A, A, None, None, None) == -1
    assert f(A, ODD, A, 1, 9, 4096, A, A, None, None, None) == -3
    assert f(A, None, A, 1, 9, 4096, A, A, A + 2, None, None) == -3     # logprob: fp32 alignment
    assert f(A, None, A, 1, 9, 4096, A, A, None, A + 2, None) == -3     # kv_len: int32 alignment


def test_head_greedy_argument_errors(xv):
    f = xv.lib().xv_head_greedy_accept
    wsb = xv.xv_head_greedy_workspace_bytes(1, 9, 4096)
    assert wsb == 256 + 16 * 9 * 256
    assert xv.xv_head_greedy_workspace_bytes(0, 9, 4096) == 256
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("xa", A), ("wa", A), ("ya", A), ("la", A), ("xb", A), ("wb", A), ("yb", A), ("lb", A),
        ("draft", A), ("ids", A), ("nk", A), ("lp", None), ("kv", None), ("ws", A), ("wsb", wsb),
        ("B", 1), ("T", 9), ("N", 4096), ("K", 6144), ("st", None))]
    assert f(*args(B=0)) == 0                          # nothing to do
    assert f(*args(T=0)) == -2 and f(*args(T=17)) == -2 and f(*args(B=-1)) == -2
    assert f(*args(N=4100)) == -2 and f(*args(K=6100)) == -2 and f(*args(N=0)) == -2
    assert f(*args(xa=None)) == -1 and f(*args(lb=None)) == -1 and f(*args(ws=None)) == -1
    assert f(*args(draft=None)) == -1 and f(*args(nk=None)) == -1
    assert f(*args(wb=MIS)) == -3 and f(*args(ws=A + 4)) == -3 and f(*args(lp=A + 2)) == -3
    assert f(*args(wsb=wsb - 1)) == -4


def test_embed_and_split_argument_errors(xv):
    e = xv.lib().xv_embed_rows
    assert e(A, A, 0, 4096, 5120, A, None) == 0
    assert e(A, A, 9, 0, 5120, A, None) == -2 and e(A, A, 9, 4096, 5124, A, None) == -2
    assert e(None, A, 9, 4096, 5120, A, None) == -1 and e(A, A, 9, 4096, 5120, None, None) == -1
    assert e(MIS, A, 9, 4096, 5120, A, None) == -3 and e(A, A + 2, 9, 4096, 5120, A, None) == -3
    s = xv.lib().xv_split_projections
    ok = dict(M=9, N1=10240, N2=17408, Hk=16, Hv=48, dk=128, dv=128, Hq=24, Hkv=4, d=256)

    def call(ptrs=None, **kw):
        a = dict(ok); a.update(kw)
        p = [A] * 10 if ptrs is None else ptrs
        return s(p[0], p[1], a["M"], a["N1"], a["N2"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                 a["Hq"], a["Hkv"], a["d"], *p[2:], None)

    assert call(M=0) == 0
    assert call(dk=96) == -2 and call(dv=12) == -2 and call(d=20) == -2
    assert call(N1=10232) == -2                       # too few columns for q, k, v
    assert call(N2=8280) == -2                        # 6144 + 2048 + 96 = 8288 needed
    assert call(N1=10244) == -2                       # rows must stay 16-byte aligned
    assert call(ptrs=[A] * 9 + [None]) == -1
    assert call(ptrs=[MIS] + [A] * 9) == -3
    assert call(ptrs=[A] * 5 + [A + 2] + [A] * 4) == -3  # a: fp32 alignment


def test_product_path_does_not_touch_the_oracle():
    """No product file imports, loads or names the oracle package."""
    pkg = os.path.join(ROOT, "bit_exact_speculative_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn
                assert "liboracle" not in src and "xo_" not in src, fn
