"""xv_attn_verify_rows on the GPU: oracle parity, KV append bytes, verify rows ==
decode rows bit for bit, and independence from capacity and workspace size."""
import numpy as np
import pytest
import torch

import oracle
from bit_exact_speculative_amd.inputs import f32_to_bf16_bits, random_bf16
from tests.gpu_util import OUT_MAX_REL, OUT_REL_L2, max_rel, rel_l2, same_bits, workload

pytestmark = pytest.mark.gpu
NAN = 0x7FC0


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _case(seed, B, T, Hq, Hkv, d, L0, Lmax):
    rng = np.random.default_rng(seed)
    q = random_bf16(rng, (B, T, Hq, d))
    kn = random_bf16(rng, (B, T, Hkv, d)); vn = random_bf16(rng, (B, T, Hkv, d))
    kc = np.full((B, Hkv, Lmax, d), NAN, np.uint16); vc = np.full_like(kc, NAN)
    for bb in range(B):
        kc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
        vc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
    return q, kn, vn, kc, vc, np.asarray(L0, np.int32)


class Dev:
    def __init__(self, q, kn, vn, kc, vc, L0):
        from bit_exact_speculative_amd.layer import dev, dev_bf16
        self.q = dev_bf16(q, "cuda"); self.kn = dev_bf16(kn, "cuda"); self.vn = dev_bf16(vn, "cuda")
        self.kc0 = dev_bf16(kc, "cuda"); self.vc0 = dev_bf16(vc, "cuda")
        self.L0 = dev(L0, "cuda")
        self.d = q.shape[3]


def _run(D, q, kn, vn, kc, vc, kv_len, ws_extra=0):
    B, T, Hq, d = q.shape
    Lmax = kc.shape[2]
    o = torch.empty((B, T, Hq, d), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((B, T, Hq, d), dtype=torch.float32, device="cuda")
    # partials NaN (each call writes what it reads), arrival counters zero; ws_extra: a larger buffer
    ws = _xv().xv_attn_workspace(B, T, Hq, d, Lmax, fill=float("nan"))
    if ws_extra:
        ws = torch.cat([ws, torch.full(((ws_extra + 15) // 16 * 4,), float("nan"), device="cuda")])
    _xv().xv_attn_verify_rows(q, kn, vn, kc, vc, kv_len, o, o32, ws, 1.0 / d ** 0.5)
    return o, o32


def _verify(D, Lmax_extra=0, ws_extra=0):
    kc = D.kc0.clone(); vc = D.vc0.clone()
    if Lmax_extra:
        B, Hkv, L, d = kc.shape
        pad = torch.full((B, Hkv, Lmax_extra, d), 1.0, dtype=torch.bfloat16, device="cuda")
        kc = torch.cat([kc, pad], 2).contiguous(); vc = torch.cat([vc, pad], 2).contiguous()
    o, o32 = _run(D, D.q, D.kn, D.vn, kc, vc, D.L0.clone(), ws_extra)
    return o, o32, kc, vc


def _decode(D):
    B, T = D.q.shape[:2]
    kc = D.kc0.clone(); vc = D.vc0.clone(); kv = D.L0.clone()
    os_, o32s = [], []
    for t in range(T):
        sl = slice(t, t + 1)
        o, o32 = _run(D, D.q[:, sl].contiguous(), D.kn[:, sl].contiguous(), D.vn[:, sl].contiguous(),
                      kc, vc, kv)
        kv += 1                                     # the decode step keeps its row
        os_.append(o[:, 0]); o32s.append(o32[:, 0])
    return torch.stack(os_, 1), torch.stack(o32s, 1), kc, vc


CASES = [
    # B, T, Hq, Hkv, d, L0s
    (1, 5, 4, 1, 64, [128]),
    (1, 9, 24, 4, 256, [640]),
    (2, 9, 6, 2, 128, [255, 256]),          # rows straddle a chunk boundary
    (3, 16, 8, 1, 64, [0, 1, 247]),         # empty cache, 1 position, 128 pairs per group
    (1, 1, 24, 4, 256, [511]),              # decode shape
    (2, 4, 12, 3, 256, [1000, 31]),
    (1, 16, 16, 1, 128, [300]),             # 256 pairs per group (16 tiles)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_attn_matches_oracle_and_appends(case):
    B, T, Hq, Hkv, d, L0 = case
    Lmax = max(L0) + T + 5
    arrs = _case(sum(L0) + T, B, T, Hq, Hkv, d, L0, Lmax)
    D = Dev(*arrs)
    o, o32, kc, vc = _verify(D)
    torch.cuda.synchronize()
    q, kn, vn, kc0, vc0, L0a = arrs
    ref = oracle.attn(q, kn, vn, kc0, vc0, L0a, 1.0 / d ** 0.5)
    o32h = o32.cpu().numpy()
    assert np.all(np.isfinite(o32h))
    assert max_rel(o32h, ref) <= OUT_MAX_REL and rel_l2(o32h, ref) <= OUT_REL_L2
    from bit_exact_speculative_amd.layer import host_bits
    assert np.array_equal(host_bits(o), f32_to_bf16_bits(o32h))
    # append: rows L0..L0+T-1 hold the new rows; every other slot is untouched
    kch, vch = host_bits(kc), host_bits(vc)
    for bb in range(B):
        n = L0[bb]
        assert np.array_equal(kch[bb, :, n:n + T], kn[bb].transpose(1, 0, 2))
        assert np.array_equal(vch[bb, :, n:n + T], vn[bb].transpose(1, 0, 2))
        assert np.array_equal(kch[bb, :, :n], kc0[bb, :, :n])
        assert np.all(kch[bb, :, n + T:] == NAN) and np.all(vch[bb, :, n + T:] == NAN)


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_attn_verify_rows_equal_decode_rows(case):
    B, T, Hq, Hkv, d, L0 = case
    Lmax = max(L0) + T
    D = Dev(*_case(7 + sum(L0) + T, B, T, Hq, Hkv, d, L0, Lmax))
    o, o32, kc, vc = _verify(D)
    od, o32d, kcd, vcd = _decode(D)
    torch.cuda.synchronize()
    assert same_bits(o32, o32d) and same_bits(o, od)
    assert same_bits(kc, kcd) and same_bits(vc, vcd)


@pytest.mark.parametrize("T", [1, 2, 8, 9, 12, 16])
def test_attn_verify_equals_decode_every_T(T):
    D = Dev(*_case(40 + T, 1, T, 8, 1, 128, [300], 300 + T))
    o, o32, kc, vc = _verify(D)
    od, o32d, kcd, vcd = _decode(D)
    torch.cuda.synchronize()
    assert same_bits(o32, o32d) and same_bits(kc, kcd)


def test_attn_capacity_and_workspace_invariance():
    D = Dev(*_case(77, 2, 9, 12, 2, 256, [700, 260], 709))
    o, o32, _, _ = _verify(D)
    for extra, wsx in ((0, 4096), (300, 0), (4096 * 8, 1 << 20)):
        o2, o322, _, _ = _verify(D, Lmax_extra=extra, ws_extra=wsx)
        assert same_bits(o32, o322) and same_bits(o, o2), (extra, wsx)


@pytest.mark.parametrize("case", [(1, 9, 24, 4, 256, [640]), (2, 16, 8, 1, 64, [0, 700]),
                                  (1, 5, 6, 2, 128, [257]), (3, 1, 24, 4, 256, [5, 300, 1000])],
                         ids=lambda c: str(c))
@pytest.mark.parametrize("grid", [128, 1024])
def test_attn_wide_and_tile_kernels_agree(case, grid):
    """The partial kernels form the same numbers: the same rows at a small capacity (few
    (chunk, KV head, request) workgroups: the tile kernel) and at capacities that give at least
    128 of them (the wide kernel) or 1024 (the persistent streaming kernel, up to 64 pairs)."""
    B, T, Hq, Hkv, d, L0 = case
    C = _xv().xv_attn_chunk_tokens()
    Lmax = max(L0) + T
    assert B * Hkv * -(-Lmax // C) < 128                     # small capacity: tile kernel
    D = Dev(*_case(123 + sum(L0), B, T, Hq, Hkv, d, L0, Lmax))
    o, o32, kc, vc = _verify(D)
    extra = -(-grid // (B * Hkv)) * C - Lmax                 # large capacity
    o2, o322, kc2, vc2 = _verify(D, Lmax_extra=extra)
    torch.cuda.synchronize()
    assert same_bits(o32, o322) and same_bits(o, o2)
    assert same_bits(kc, kc2[:, :, :Lmax]) and same_bits(vc, vc2[:, :, :Lmax])


def test_attn_stream_group_partials_agree_with_chunk_partials():
    """A 40,000-position row (157 chunks, 20 groups of 8): at a capacity that takes the wide
    kernel the combine folds the chunk partials in two levels; at one that takes the
    streaming kernel (65,536 positions: 32 workgroups per KV head, fewer than twice the
    groups) the kernel folds each group's chunks itself and the combine folds the groups.
    Every output bit and the appended rows agree, and the outputs meet the oracle's bounds."""
    B, T, Hq, Hkv, d, L0 = 1, 9, 24, 4, 256, [40000]
    C = _xv().xv_attn_chunk_tokens()
    Lmax = max(L0) + T
    assert 128 <= B * Hkv * -(-Lmax // C) < 1024            # the wide kernel
    arrs = _case(4242, B, T, Hq, Hkv, d, L0, Lmax)
    D = Dev(*arrs)
    o, o32, kc, vc = _verify(D)
    o2, o322, kc2, vc2 = _verify(D, Lmax_extra=65536 - Lmax)   # the streaming kernel, group partials
    torch.cuda.synchronize()
    assert same_bits(o32, o322) and same_bits(o, o2)
    assert same_bits(kc, kc2[:, :, :Lmax]) and same_bits(vc, vc2[:, :, :Lmax])
    q, kn, vn, kc0, vc0, L0a = arrs
    ref = oracle.attn(q, kn, vn, kc0, vc0, L0a, 1.0 / d ** 0.5)
    o32h = o322.cpu().numpy()
    assert max_rel(o32h, ref) <= OUT_MAX_REL and rel_l2(o32h, ref) <= OUT_REL_L2


def test_attn_tile_value_dim_parts_agree():
    """At d = 256 a tile workgroup forms half of a chunk's output dims while that grid fits
    the chip, all of them beyond (capacity 2304: 9 chunks x 4 KV heads x 4 tiles x 2 halves =
    288 workgroups, more than 256 CUs): the same bits either way."""
    B, T, Hq, Hkv, d, L0 = 1, 9, 24, 4, 256, [640]
    Lmax = max(L0) + T
    D = Dev(*_case(321, B, T, Hq, Hkv, d, L0, Lmax))
    o, o32, kc, vc = _verify(D)
    o2, o322, kc2, vc2 = _verify(D, Lmax_extra=2304 - Lmax)
    torch.cuda.synchronize()
    assert same_bits(o32, o322) and same_bits(o, o2)
    assert same_bits(kc, kc2[:, :, :Lmax]) and same_bits(vc, vc2[:, :, :Lmax])


def test_attn_batch_invariance():
    D = Dev(*_case(88, 8, 9, 24, 4, 256, [560, 740, 600, 611, 699, 573, 720, 640], 749))
    o, o32, kc, vc = _verify(D)
    for bb in range(8):
        sl = slice(bb, bb + 1)
        o1, o321 = _run(D, D.q[sl].contiguous(), D.kn[sl].contiguous(), D.vn[sl].contiguous(),
                        D.kc0[sl].clone(), D.vc0[sl].clone(), D.L0[sl].clone())
        assert same_bits(o321[0], o32[bb]) and same_bits(o1[0], o[bb]), bb


def test_attn_medium_context_vs_oracle():
    inp, _ = workload("medium", gemm=False, head=False)
    D = Dev(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0)
    o, o32, _, _ = _verify(D)
    torch.cuda.synchronize()
    ref = oracle.attn(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0, 1.0 / 16)
    assert max_rel(o32.cpu().numpy(), ref) <= OUT_MAX_REL and rel_l2(o32.cpu().numpy(), ref) <= OUT_REL_L2


def test_attn_repeatable_and_two_streams():
    D = Dev(*_case(99, 8, 9, 24, 4, 256, [600] * 8, 609))
    o, o32, _, _ = _verify(D)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(40):
        with torch.cuda.stream(s1 if i % 2 == 0 else s2):
            outs.append(_verify(D)[1])
    torch.cuda.synchronize()
    for x in outs:
        assert same_bits(x, o32)
