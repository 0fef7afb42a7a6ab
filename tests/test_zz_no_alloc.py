"""xv_attn_verify_rows_noalloc (the library's own partials buffer, no allocation) against
xv_attn_verify_rows with a caller workspace: every output bit, on calls in a row where
the later call is smaller (the buffer keeps the earlier call's contents)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import same_bits

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _case(seed, B, T, Hq, Hkv, d, L0s, Lmax):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).cuda()
    q = bf(B, T, Hq, d)
    kn, vn = bf(B, T, Hkv, d), bf(B, T, Hkv, d)
    kc, vc = bf(B, Hkv, Lmax, d), bf(B, Hkv, Lmax, d)
    kv = torch.tensor(L0s, dtype=torch.int32).cuda()
    return q, kn, vn, kc, vc, kv


def _both(case):
    xv = _xv()
    q, kn, vn, kc, vc, kv = case
    B, T, Hq, d = q.shape
    Lmax = kc.shape[2]
    wsb = xv.xv_attn_workspace_bytes(B, T, Hq, d, Lmax)
    assert wsb <= 32 << 20
    ws = xv.xv_attn_workspace(B, T, Hq, d, Lmax)
    kc1, vc1, kc2, vc2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    o1 = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    o321 = torch.empty((B, T, Hq, d), dtype=torch.float32, device="cuda")
    o2, o322 = torch.empty_like(o1), torch.empty_like(o321)
    xv.xv_attn_verify_rows(q, kn, vn, kc1, vc1, kv, o1, o321, ws)
    xv.xv_attn_verify_rows_noalloc(q, kn, vn, kc2, vc2, kv, o2, o322)
    torch.cuda.synchronize()
    return (o1, o321, kc1, vc1), (o2, o322, kc2, vc2)


# (B, T, Hq, Hkv, d, L0 per request, Lmax): the tile split (one request), the wide split
# (eight requests, five chunks of capacity), the streaming split (a long context with few
# query heads), a small head dim; each pair of calls: the larger first
CASES = [
    [(1, 9, 24, 4, 256, [640], 700), (1, 5, 24, 4, 256, [200], 260)],
    [(8, 9, 24, 4, 256, [560 + 23 * i for i in range(8)], 1028), (2, 3, 24, 4, 256, [100, 37], 160)],
    [(1, 2, 8, 4, 256, [70000], 70100), (1, 1, 8, 4, 256, [3000], 3100)],
    [(1, 16, 4, 1, 64, [2000], 2100), (1, 1, 4, 1, 64, [0], 8)],
]


@pytest.mark.parametrize("pair", range(len(CASES)))
def test_noalloc_equals_workspace_call(pair):
    for i, (B, T, Hq, Hkv, d, L0s, Lmax) in enumerate(CASES[pair]):
        ref, got = _both(_case(9000 + 10 * pair + i, B, T, Hq, Hkv, d, L0s, Lmax))
        for a, b in zip(ref, got):
            assert same_bits(a, b), (pair, i)


def test_noalloc_rejects_oversize_before_launch():
    xv = _xv()
    case = _case(9100, 1, 9, 24, 4, 256, [640], 700)
    q, kn, vn, kc, vc, kv = case
    big_c = torch.empty((1, 4, 40000, 256), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((1, 9, 24, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(xv.XvError):
        xv.xv_attn_verify_rows_noalloc(q, kn, vn, big_c, big_c, kv, o)
    torch.cuda.synchronize()
