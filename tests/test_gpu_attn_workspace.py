"""The attention workspace's arrival counters (its first 4096 bytes): every call leaves them zero,
so one buffer zeroed once serves a sequence of calls of different shapes, each giving the bits
of a call with a fresh workspace; the tile workgroups that fold their rows and the separate
combine launch are both exercised (xv_attn_verify_rows and xv_gdn_attn_verify)."""
import torch
import pytest

from tests.gpu_util import same_bits

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _case(seed, B, T, Hq, Hkv, d, L0, Lmax):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = lambda *s: torch.randn(s, generator=g, device="cuda").to(torch.bfloat16)
    return (bf(B, T, Hq, d), bf(B, T, Hkv, d), bf(B, T, Hkv, d), bf(B, Hkv, Lmax, d), bf(B, Hkv, Lmax, d),
            torch.tensor(L0, dtype=torch.int32, device="cuda"))


def _call(case, ws):
    q, kn, vn, kc0, vc0, kv = case
    B, T, Hq, d = q.shape
    kc, vc = kc0.clone(), vc0.clone()
    o = torch.full((B, T, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o32 = torch.full((B, T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    _xv().xv_attn_verify_rows(q, kn, vn, kc, vc, kv, o, o32, ws)
    torch.cuda.synchronize()
    return o, o32, kc, vc


# (B, T, Hq, Hkv, d, L0, Lmax): the per-tile split (folding in its launch) at several sizes, the
# wide split (a combine launch), and the per-tile split again after them
SHAPES = [
    (1, 9, 24, 4, 256, [640], 700),
    (2, 5, 8, 2, 128, [300, 17], 400),
    (8, 9, 24, 4, 256, [560 + 23 * i for i in range(8)], 1028),
    (1, 16, 4, 1, 64, [2000], 2100),
    (1, 3, 24, 4, 256, [5], 20),
    (1, 9, 24, 4, 256, [2183], 2471),
]


def test_one_workspace_serves_calls_of_every_shape():
    xv = _xv()
    need = max(xv.xv_attn_workspace_bytes(B, T, Hq, d, Lmax) for B, T, Hq, Hkv, d, L0, Lmax in SHAPES)
    shared = torch.zeros(((need + 15) // 16 * 4,), dtype=torch.float32, device="cuda")
    for rep in range(2):
        for i, (B, T, Hq, Hkv, d, L0, Lmax) in enumerate(SHAPES):
            case = _case(100 * rep + i, B, T, Hq, Hkv, d, L0, Lmax)
            got = _call(case, shared)
            ref = _call(case, xv.xv_attn_workspace(B, T, Hq, d, Lmax))
            for x, y, name in zip(got, ref, ("o", "o32", "k_cache", "v_cache")):
                assert same_bits(x, y), (rep, i, name)
            assert not torch.isnan(got[1]).any(), (rep, i)
            counters = shared[:xv.ATTN_COUNTER_BYTES // 4].view(torch.int32)
            assert int(counters.abs().sum()) == 0, (rep, i)
