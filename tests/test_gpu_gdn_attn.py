"""xv_gdn_attn_verify on the GPU: GDN and attention in one call give every bit of the
two calls it stands for (xv_gdn_verify or xv_gdn_verify_after, then
xv_attn_verify_rows), whether the library runs them in one launch or in two."""
import numpy as np
import pytest
import torch

from bit_exact_speculative_amd.inputs import random_bf16, random_gdn
from tests.gpu_util import same_bits

pytestmark = pytest.mark.gpu
NAN = 0x7FC0


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _inputs(seed, B, T, Hk, Hv, dk, dv, Hq, Hkv, d, L0, Lmax, Tp):
    from bit_exact_speculative_amd.layer import dev, dev_bf16
    rng = np.random.default_rng(seed)
    g = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    gp = random_gdn(rng, B, Tp, Hk, Hv, dk, dv)
    cur = dict(q=dev_bf16(g["q"], "cuda"), k=dev_bf16(g["k"], "cuda"), v=dev_bf16(g["v"], "cuda"),
               a=dev(g["a"], "cuda"), b=dev(g["b"], "cuda"))
    prev = dict(k=dev_bf16(gp["k"], "cuda"), v=dev_bf16(gp["v"], "cuda"), a=dev(gp["a"], "cuda"),
                b=dev(gp["b"], "cuda"))
    S = [torch.from_numpy((rng.standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)).cuda()
         for _ in range(2)]
    kc = np.full((B, Hkv, Lmax, d), NAN, np.uint16)
    vc = np.full_like(kc, NAN)
    for bb in range(B):
        kc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
        vc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
    att = dict(q=dev_bf16(random_bf16(rng, (B, T, Hq, d)), "cuda"),
               kn=dev_bf16(random_bf16(rng, (B, T, Hkv, d)), "cuda"),
               vn=dev_bf16(random_bf16(rng, (B, T, Hkv, d)), "cuda"),
               kc=dev_bf16(kc, "cuda"), vc=dev_bf16(vc, "cuda"),
               L0=torch.from_numpy(np.asarray(L0, np.int32)).cuda())
    nk = torch.from_numpy(rng.integers(0, Tp + 1, size=B).astype(np.int32)).cuda()
    nk[0] = Tp                                        # one request keeps every previous row
    return cur, prev, S, att, nk


def _outs(B, T, Hv, dv, Hq, d, dk, Lmax):
    e = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda")
    f = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    return dict(o=e(B, T, Hv, dv), o32=f(B, T, Hv, dv), oa=e(B, T, Hq, d), oa32=f(B, T, Hq, d),
                kept=f(B, Hv, dk, dv), out=f(B, Hv, dk, dv),
                ws=_xv().xv_attn_workspace(B, T, Hq, d, Lmax, fill=float("nan")))


# (B, T, Hk, Hv, dk, dv, Hq, Hkv, d, L0, Lmax, Tp).  The first three and the last fit one launch:
# 8 * ceil(items / 8) tile workgroups (items = B Hkv ceil(Lmax/256) ceil(Hq/Hkv T/16) DS)
# plus B Hv dv / 64 (or / 32) GDN workgroups at most 256; e.g. 160 + 96 for the first.
CASES = [
    (1, 9, 16, 48, 128, 128, 24, 4, 256, [640], 1171, 9),
    (2, 5, 2, 4, 64, 64, 8, 2, 128, [300, 17], 600, 3),
    (1, 3, 1, 2, 128, 96, 4, 1, 64, [40], 100, 16),
    (8, 9, 16, 48, 128, 128, 24, 4, 256, [640, 1, 300, 255, 256, 257, 512, 700], 1024, 9),   # two launches
    # 10 chunks: 320 tile workgroups of halves would not fit beside GDN, 160 of whole chunks do
    (1, 9, 16, 48, 128, 128, 24, 4, 256, [2183], 2471, 9),
]


@pytest.mark.parametrize("case", CASES, ids=["short", "small", "dv96", "batch8", "medium"])
@pytest.mark.parametrize("after", [False, True])
def test_gdn_attn_equals_the_two_calls(case, after):
    B, T, Hk, Hv, dk, dv, Hq, Hkv, d, L0, Lmax, Tp = case
    cur, prev, S, att, nk = _inputs(sum(L0) + T + dv, *case)
    scale = 1.0 / d ** 0.5
    xv = _xv()
    # the two calls
    r = _outs(B, T, Hv, dv, Hq, d, dk, Lmax)
    kc_r, vc_r, kv_r = att["kc"].clone(), att["vc"].clone(), att["L0"].clone()
    if after:
        xv.xv_gdn_verify_after(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], prev["k"], prev["v"],
                               prev["a"], prev["b"], nk, S[0], S[1], r["kept"], r["out"], r["o"], r["o32"])
    else:
        xv.xv_gdn_verify(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], S[0], r["out"], r["o"], r["o32"])
    xv.xv_attn_verify_rows(att["q"], att["kn"], att["vn"], kc_r, vc_r, kv_r, r["oa"], r["oa32"], r["ws"], scale)
    # one call
    f = _outs(B, T, Hv, dv, Hq, d, dk, Lmax)
    kc_f, vc_f, kv_f = att["kc"].clone(), att["vc"].clone(), att["L0"].clone()
    pv = (prev["k"], prev["v"], prev["a"], prev["b"], nk, S[1], f["kept"]) if after else None
    xv.xv_gdn_attn_verify(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], S[0], f["out"], f["o"],
                          att["q"], att["kn"], att["vn"], kc_f, vc_f, kv_f, f["oa"], f["ws"], scale,
                          o32=f["o32"], o_attn32=f["oa32"], prev=pv)
    torch.cuda.synchronize()
    assert same_bits(f["o"], r["o"]) and same_bits(f["o32"], r["o32"]) and same_bits(f["out"], r["out"])
    if after:
        assert same_bits(f["kept"], r["kept"])
    assert same_bits(f["oa"], r["oa"]) and same_bits(f["oa32"], r["oa32"])
    assert same_bits(kc_f, kc_r) and same_bits(vc_f, vc_r) and torch.equal(kv_f, kv_r)
    assert not torch.isnan(f["o32"]).any() and not torch.isnan(f["oa32"]).any()


def test_gdn_attn_repeatable():
    """The same call 50 times: the same bits every time (no dependence on which
    workgroups of the shared launch run first)."""
    case = CASES[0]
    B, T, Hk, Hv, dk, dv, Hq, Hkv, d, L0, Lmax, Tp = case
    cur, prev, S, att, nk = _inputs(77, *case)
    xv = _xv()
    ref = None
    for _ in range(50):
        f = _outs(B, T, Hv, dv, Hq, d, dk, Lmax)
        kc, vc, kv = att["kc"].clone(), att["vc"].clone(), att["L0"].clone()
        xv.xv_gdn_attn_verify(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], S[0], f["out"], f["o"],
                              att["q"], att["kn"], att["vn"], kc, vc, kv, f["oa"], f["ws"],
                              o32=f["o32"], o_attn32=f["oa32"],
                              prev=(prev["k"], prev["v"], prev["a"], prev["b"], nk, S[1], f["kept"]))
        got = [f["o32"], f["out"], f["kept"], f["oa32"], kc]
        if ref is None:
            ref = got
        else:
            assert all(same_bits(x, y) for x, y in zip(got, ref))
