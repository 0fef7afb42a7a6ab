"""len_bound on the attention calls: a launch sized for an upper bound on kv_len + T instead of
the cache capacity gives the bits of the capacity-sized launch (outputs, appended rows,
lengths), for bounds from max(kv_len) + T up to the capacity; at a 262,144-position capacity
with rows of a few hundred positions the bound switches the launch from the streaming
kernel to the per-tile split, and xv_gdn_attn_verify to one shared launch."""
import numpy as np
import pytest
import torch

from bit_exact_speculative_amd.inputs import random_gdn
from tests.gpu_util import same_bits

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _attn_inputs(seed, B, T, Hq, Hkv, d, L0, Lmax):
    """Caches hold random rows below L0[b] and NaN above (positions that must not be read)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.full((B, Hkv, Lmax, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    for b in range(B):
        if L0[b]:
            kc[b, :, :L0[b]] = bf(Hkv, L0[b], d)
            vc[b, :, :L0[b]] = bf(Hkv, L0[b], d)
    kv = torch.tensor(L0, dtype=torch.int32, device="cuda")
    return bf(B, T, Hq, d), bf(B, T, Hkv, d), bf(B, T, Hkv, d), kc, vc, kv


def _bounds(L0, T, Lmax):
    lo = max(L0) + T
    return sorted({b for b in (0, lo, lo + 1, lo + 255, lo + 777, Lmax) if b == 0 or lo <= b <= Lmax})


def _run(inp, lb, B, T, Hq, d, Lmax, noalloc=False):
    xv = _xv()
    q, kn, vn, kc0, vc0, kv0 = inp
    kc, vc, kv = kc0.clone(), vc0.clone(), kv0.clone()
    o = torch.full((B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o32 = torch.full((B, T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        xv.xv_attn_verify_rows_noalloc(q, kn, vn, kc, vc, kv, o, o32, len_bound=lb)
    else:
        ws = xv.xv_attn_workspace(B, T, Hq, d, Lmax, fill=float("nan"))
        xv.xv_attn_verify_rows(q, kn, vn, kc, vc, kv, o, o32, ws, len_bound=lb)
    torch.cuda.synchronize()
    return o, o32, kc, vc, kv


# (B, T, Hq, Hkv, d, L0, Lmax)
CASES = [
    (1, 9, 24, 4, 256, [300], 262144),        # streaming kernel without a bound, per-tile with one
    (1, 9, 24, 4, 256, [4000], 262144),
    (1, 1, 24, 4, 256, [0], 262144),          # an empty cache
    (2, 5, 8, 2, 128, [700, 17], 30000),
    (8, 9, 24, 4, 256, [640, 1, 300, 255, 256, 257, 512, 700], 262144),
    (1, 16, 4, 1, 64, [4984], 5000),          # the bound reaches the capacity
    (3, 7, 16, 4, 128, [2000, 2500, 1900], 65536),
]


@pytest.mark.parametrize("case", CASES, ids=["short", "4k", "empty", "small", "batch8", "full", "mid"])
def test_attn_len_bound_same_bits(case):
    B, T, Hq, Hkv, d, L0, Lmax = case
    inp = _attn_inputs(sum(L0) + 31 * T + d, *case)
    ref = _run(inp, 0, B, T, Hq, d, Lmax)
    assert not torch.isnan(ref[1]).any()
    for lb in _bounds(L0, T, Lmax)[1:]:
        got = _run(inp, lb, B, T, Hq, d, Lmax)
        for x, y, name in zip(got, ref, ("o", "o32", "k_cache", "v_cache", "kv_len")):
            assert same_bits(x, y), (name, lb)


@pytest.mark.parametrize("case", [(1, 9, 24, 4, 256, [300], 3000), (2, 5, 8, 2, 128, [700, 17], 30000)],
                         ids=["short", "small"])
def test_attn_noalloc_len_bound_same_bits(case):
    B, T, Hq, Hkv, d, L0, Lmax = case
    inp = _attn_inputs(5 + sum(L0), *case)
    ref = _run(inp, 0, B, T, Hq, d, Lmax)
    for lb in _bounds(L0, T, Lmax):
        got = _run(inp, lb, B, T, Hq, d, Lmax, noalloc=True)
        for x, y, name in zip(got, ref, ("o", "o32", "k_cache", "v_cache", "kv_len")):
            assert same_bits(x, y), (name, lb)


@pytest.mark.parametrize("after", [False, True])
@pytest.mark.parametrize("L0,Lmax", [([640], 262144), ([300], 32768), ([5000], 262144)],
                         ids=["short_262144", "short_32768", "5k_262144"])
def test_gdn_attn_len_bound_same_bits(L0, Lmax, after):
    """xv_gdn_attn_verify with and without a bound, against GDN then attention (no bound)."""
    from bit_exact_speculative_amd.layer import dev, dev_bf16
    xv = _xv()
    B, T, Hk, Hv, dk, dv, Hq, Hkv, d, Tp = 1, 9, 16, 48, 128, 128, 24, 4, 256, 9
    rng = np.random.default_rng(Lmax + L0[0])
    g, gp = random_gdn(rng, B, T, Hk, Hv, dk, dv), random_gdn(rng, B, Tp, Hk, Hv, dk, dv)
    cur = [dev_bf16(g["q"], "cuda"), dev_bf16(g["k"], "cuda"), dev_bf16(g["v"], "cuda"),
           dev(g["a"], "cuda"), dev(g["b"], "cuda")]
    S = [torch.from_numpy((rng.standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)).cuda()
         for _ in range(2)]
    nk = torch.tensor([5], dtype=torch.int32, device="cuda")
    att = _attn_inputs(17, B, T, Hq, Hkv, d, L0, Lmax)
    scale = 1.0 / d ** 0.5
    f32 = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")

    def outs():
        return dict(o=torch.full((B, T, Hv, dv), float("nan"), dtype=torch.bfloat16, device="cuda"),
                    o32=f32(B, T, Hv, dv), kept=f32(B, Hv, dk, dv), out=f32(B, Hv, dk, dv),
                    oa=torch.full((B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda"),
                    oa32=f32(B, T, Hq, d), ws=xv.xv_attn_workspace(B, T, Hq, d, Lmax),
                    kc=att[3].clone(), vc=att[4].clone(), kv=att[5].clone())

    prev = None
    if after:
        gpk = [dev_bf16(gp["k"], "cuda"), dev_bf16(gp["v"], "cuda"), dev(gp["a"], "cuda"), dev(gp["b"], "cuda")]
    r = outs()
    if after:
        xv.xv_gdn_verify_after(*cur, *gpk, nk, S[0], S[1], r["kept"], r["out"], r["o"], r["o32"])
    else:
        xv.xv_gdn_verify(*cur, S[0], r["out"], r["o"], r["o32"])
    xv.xv_attn_verify_rows(att[0], att[1], att[2], r["kc"], r["vc"], r["kv"], r["oa"], r["oa32"], r["ws"], scale)
    torch.cuda.synchronize()
    for lb in (0, L0[0] + T, L0[0] + T + 1000):
        f = outs()
        prev = (*gpk, nk, S[1], f["kept"]) if after else None
        xv.xv_gdn_attn_verify(*cur, S[0], f["out"], f["o"], att[0], att[1], att[2], f["kc"], f["vc"], f["kv"],
                              f["oa"], f["ws"], scale, o32=f["o32"], o_attn32=f["oa32"], prev=prev,
                              len_bound=lb)
        torch.cuda.synchronize()
        keys = ["o", "o32", "out", "oa", "oa32", "kc", "vc", "kv"] + (["kept"] if after else [])
        for k in keys:
            assert same_bits(f[k], r[k]), (k, lb)
