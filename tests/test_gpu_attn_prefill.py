"""xv_attn_prefill on the GPU: P prompt rows at once give every bit of the same rows
formed as decode / verify rows (xv_attn_verify_rows in steps, the length advanced
between steps), the same appended cache rows, and oracle parity."""
import numpy as np
import pytest
import torch

import oracle
from bit_exact_speculative_amd.inputs import random_bf16
from tests.gpu_util import OUT_MAX_REL, max_rel, same_bits

pytestmark = pytest.mark.gpu
NAN = 0x7FC0


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _case(seed, B, P, Hq, Hkv, d, L0, Lmax):
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(seed)
    q = random_bf16(rng, (B, P, Hq, d), 2.0)
    kn = random_bf16(rng, (B, P, Hkv, d)); vn = random_bf16(rng, (B, P, Hkv, d))
    kc = np.full((B, Hkv, Lmax, d), NAN, np.uint16); vc = np.full_like(kc, NAN)
    for bb in range(B):
        kc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
        vc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
    host = (q, kn, vn, kc, vc)
    dev = [dev_bf16(a, "cuda") for a in host]
    return host, dev, torch.tensor(L0, dtype=torch.int32, device="cuda")


def _steps(dev, kv0, T):
    """The rows as verify steps of T rows (decode arithmetic), the length advanced after each."""
    q, kn, vn, kc, vc = [t.clone() for t in dev]
    B, P, Hq, d = q.shape
    Lmax = kc.shape[2]
    kv = kv0.clone()
    o = torch.empty((B, P, Hq, d), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((B, P, Hq, d), dtype=torch.float32, device="cuda")
    for t0 in range(0, P, T):
        tt = min(T, P - t0)
        sl = slice(t0, t0 + tt)
        ws = _xv().xv_attn_workspace(B, tt, Hq, d, Lmax)
        os_ = torch.empty((B, tt, Hq, d), dtype=torch.bfloat16, device="cuda")
        o32s = torch.empty((B, tt, Hq, d), dtype=torch.float32, device="cuda")
        _xv().xv_attn_verify_rows(q[:, sl].contiguous(), kn[:, sl].contiguous(), vn[:, sl].contiguous(),
                                  kc, vc, kv, os_, o32s, ws, 1.0 / d ** 0.5)
        o[:, sl] = os_; o32[:, sl] = o32s
        kv += tt
    return o, o32, kc, vc


def _prefill(dev, kv0):
    q, kn, vn, kc, vc = [t.clone() for t in dev]
    B, P, Hq, d = q.shape
    o = torch.full((B, P, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o32 = torch.full((B, P, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    kv = kv0.clone()
    _xv().xv_attn_prefill(q, kn, vn, kc, vc, kv, o, o32, 1.0 / d ** 0.5)
    assert torch.equal(kv, kv0)                     # the length is the caller's to advance
    return o, o32, kc, vc


# (B, P, Hq, Hkv, d, L0, Lmax, verify step)
CASES = [
    (1, 45, 24, 4, 256, [640], 1024, 16),
    (2, 37, 8, 2, 128, [300, 17], 600, 9),
    (1, 300, 4, 1, 64, [0], 320, 16),
    (3, 21, 6, 3, 256, [255, 256, 257], 600, 7),
    (1, 20, 24, 4, 256, [20000], 20100, 10),
]


@pytest.mark.parametrize("case", CASES, ids=["short", "gqa4-d128", "empty-cache-d64", "chunk-edges", "long"])
def test_prefill_rows_equal_decode_rows(case):
    B, P, Hq, Hkv, d, L0, Lmax, T = case
    _, dev, kv0 = _case(sum(L0) + P + d, B, P, Hq, Hkv, d, L0, Lmax)
    o_r, o32_r, kc_r, vc_r = _steps(dev, kv0, T)
    o_p, o32_p, kc_p, vc_p = _prefill(dev, kv0)
    torch.cuda.synchronize()
    assert same_bits(o_p, o_r) and same_bits(o32_p, o32_r)
    for bb in range(B):                               # the appended rows and everything before them
        L = L0[bb] + P
        assert same_bits(kc_p[bb, :, :L], kc_r[bb, :, :L]) and same_bits(vc_p[bb, :, :L], vc_r[bb, :, :L])


def test_prefill_vs_oracle():
    B, P, Hq, Hkv, d, L0, Lmax = 1, 40, 8, 2, 128, [200], 300
    (q, kn, vn, kc, vc), dev, kv0 = _case(5, B, P, Hq, Hkv, d, L0, Lmax)
    _, o32, _, _ = _prefill(dev, kv0)
    torch.cuda.synchronize()
    ref = oracle.attn(q, kn, vn, kc, vc, np.array(L0, np.int32), 1.0 / d ** 0.5)
    assert max_rel(o32.cpu().numpy(), ref) <= OUT_MAX_REL


def test_prefill_repeatable():
    B, P, Hq, Hkv, d, L0, Lmax, _ = CASES[0]
    _, dev, kv0 = _case(9, B, P, Hq, Hkv, d, L0, Lmax)
    first = _prefill(dev, kv0)[1]
    for _ in range(20):
        assert same_bits(_prefill(dev, kv0)[1], first)
