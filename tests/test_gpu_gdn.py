"""xv_gdn_verify / xv_rollback_to_prefix on the GPU: oracle parity, verify == sequential
decode bit for bit for every T, exact rollback to every prefix, batch invariance."""
import numpy as np
import pytest
import torch

import oracle
from bit_exact_speculative_amd.inputs import f32_to_bf16_bits, random_gdn
from tests.gpu_util import OUT_MAX_REL, OUT_REL_L2, STATE_REL_L2, max_rel, rel_l2, same_bits, workload

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _dev(r):
    from bit_exact_speculative_amd.layer import dev, dev_bf16
    return dict(q=dev_bf16(r["q"], "cuda"), k=dev_bf16(r["k"], "cuda"), v=dev_bf16(r["v"], "cuda"),
                a=dev(r["a"], "cuda"), b=dev(r["b"], "cuda"))


def _verify(d, S_in):
    B, T, Hk, dk = d["q"].shape
    Hv, dv = d["v"].shape[2], d["v"].shape[3]
    S_out = torch.empty_like(S_in)
    o = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((B, T, Hv, dv), dtype=torch.float32, device="cuda")
    _xv().xv_gdn_verify(d["q"], d["k"], d["v"], d["a"], d["b"], S_in, S_out, o, o32)
    return o, o32, S_out


def _decode(d, S_in, n):
    """n single-token steps (T = 1) from S_in; per-token outputs and states."""
    S = S_in.clone()
    os_, o32s, Ss = [], [], []
    for t in range(n):
        dt = {k: v[:, t:t + 1].contiguous() for k, v in d.items()}
        o, o32, S = _verify(dt, S)
        os_.append(o[:, 0]); o32s.append(o32[:, 0]); Ss.append(S)
    return torch.stack(os_, 1), torch.stack(o32s, 1), Ss


def _case(seed, B, T, Hk, Hv, dk, dv):
    rng = np.random.default_rng(seed)
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = (rng.standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)
    return r, S0


@pytest.mark.parametrize("shape", [(1, 5, 2, 4, 64, 64), (2, 9, 2, 6, 128, 128), (1, 3, 1, 2, 64, 32),
                                   (3, 16, 2, 4, 128, 96), (1, 1, 4, 4, 128, 128)])
def test_gdn_matches_oracle(shape):
    B, T, Hk, Hv, dk, dv = shape
    r, S0 = _case(sum(shape), *shape)
    d = _dev(r)
    o, o32, S = _verify(d, torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    assert rel_l2(S.cpu().numpy(), S_ref) <= STATE_REL_L2
    assert max_rel(o32.cpu().numpy(), o_ref) <= OUT_MAX_REL
    assert rel_l2(o32.cpu().numpy(), o_ref) <= OUT_REL_L2
    from bit_exact_speculative_amd.layer import host_bits
    assert np.array_equal(host_bits(o), f32_to_bf16_bits(o32.cpu().numpy()))


def test_gdn_real_shapes_vs_oracle():
    """16 key / 48 value heads, d = 128, 9 rows, from the oracle's 32-token prefix state."""
    inp, S0 = workload("short", gemm=False, head=False)
    d = _dev(inp.gdn)
    o, o32, S = _verify(d, torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    g = inp.gdn
    o_ref, S_ref, Sall = oracle.gdn(g["q"], g["k"], g["v"], g["a"], g["b"], S0, want_all=True)
    assert rel_l2(S.cpu().numpy(), S_ref) <= STATE_REL_L2
    assert max_rel(o32.cpu().numpy(), o_ref) <= OUT_MAX_REL
    assert rel_l2(o32.cpu().numpy(), o_ref) <= OUT_REL_L2


# Large batches run the kernel with 4 lanes per state column (the library takes it when
# batch x value heads x dv / 64 reaches twice the CU count: 8 requests of 48 heads at
# dv = 128 on a 256-CU part); a request alone runs the 16-lane kernel.  The dot's
# partial tree gives both the same bits.
@pytest.mark.parametrize("dk,dv,B", [(128, 128, 8), (64, 64, 16), (128, 64, 16), (64, 128, 8)])
def test_gdn_lane_split_kernels_agree(dk, dv, B):
    T, Tp, Hk, Hv = 9, 9, 16, 48
    rng = np.random.default_rng(2000 + dk + dv + B)
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = (rng.standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    o, o32, S = _verify(d, S_in)
    # verify after a previous call (every kept count, clamped ones included) and rollback
    prev = _rows(2100 + dk + dv, B, Tp, Hk, Hv, dk, dv)
    _, _, Q = _verify(prev, S_in)
    nk_list = [(-2, 0, 1, 4, Tp, Tp + 5, 7, 2)[i % 8] for i in range(B)]
    nk = torch.tensor(nk_list, dtype=torch.int32, device="cuda")
    K, O = torch.full_like(S_in, float("nan")), torch.full_like(S_in, float("nan"))
    oa = torch.empty_like(o)
    oa32 = torch.empty_like(o32)
    _xv().xv_gdn_verify_after(d["q"], d["k"], d["v"], d["a"], d["b"], prev["k"], prev["v"], prev["a"],
                              prev["b"], nk, S_in, Q, K, O, oa, oa32)
    Sr = Q.clone()
    kv = torch.zeros((B,), dtype=torch.int32, device="cuda")
    _xv().xv_rollback_to_prefix(prev["k"], prev["v"], prev["a"], prev["b"], S_in, Sr, kv, nk)
    torch.cuda.synchronize()
    assert kv.tolist() == [min(max(n, 0), Tp) for n in nk_list]
    o_ref, S_ref, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    assert rel_l2(S.cpu().numpy(), S_ref) <= STATE_REL_L2
    assert max_rel(o32.cpu().numpy(), o_ref) <= OUT_MAX_REL
    assert rel_l2(o32.cpu().numpy(), o_ref) <= OUT_REL_L2
    for bb in range(B):
        db = {k: v[bb:bb + 1].contiguous() for k, v in d.items()}
        pb = {k: v[bb:bb + 1].contiguous() for k, v in prev.items()}
        s1 = S_in[bb:bb + 1].contiguous()
        o1, o321, S1 = _verify(db, s1)
        assert same_bits(o1[0], o[bb]) and same_bits(o321[0], o32[bb]) and same_bits(S1[0], S[bb]), bb
        K1, O1 = torch.empty_like(s1), torch.empty_like(s1)
        oa1, oa321 = torch.empty_like(o1), torch.empty_like(o321)
        _xv().xv_gdn_verify_after(db["q"], db["k"], db["v"], db["a"], db["b"], pb["k"], pb["v"], pb["a"],
                                  pb["b"], nk[bb:bb + 1].contiguous(), s1, Q[bb:bb + 1].contiguous(), K1, O1,
                                  oa1, oa321)
        Sr1 = Q[bb:bb + 1].clone()
        kv1 = torch.zeros((1,), dtype=torch.int32, device="cuda")
        _xv().xv_rollback_to_prefix(pb["k"], pb["v"], pb["a"], pb["b"], s1, Sr1, kv1, nk[bb:bb + 1].contiguous())
        torch.cuda.synchronize()
        assert same_bits(K1[0], K[bb]) and same_bits(O1[0], O[bb]), bb
        assert same_bits(oa1[0], oa[bb]) and same_bits(oa321[0], oa32[bb]), bb
        assert same_bits(Sr1[0], Sr[bb]), bb


@pytest.mark.parametrize("T", list(range(1, 17)))
def test_gdn_verify_equals_sequential_decode(T):
    r, S0 = _case(500 + T, 2, T, 2, 4, 128, 128)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    o, o32, S = _verify(d, S_in)
    od, o32d, Sd = _decode(d, S_in, T)
    torch.cuda.synchronize()
    assert same_bits(o, od) and same_bits(o32, o32d) and same_bits(S, Sd[-1])


@pytest.mark.parametrize("dk", [64, 128])
def test_rollback_every_prefix(dk):
    T = 9
    r, S0 = _case(600 + dk, 3, T, 2, 4, dk, 64)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    _, _, S_T = _verify(d, S_in)
    _, _, Sd = _decode(d, S_in, T)
    for n in range(0, T + 1):
        for mix in (False, True):
            nk = [n, n, n] if not mix else [n, (n + 4) % (T + 1), T - n]
            S_out = S_T.clone()
            kv = torch.tensor([100, 0, 7], dtype=torch.int32, device="cuda")
            n_keep = torch.tensor(nk, dtype=torch.int32, device="cuda")
            _xv().xv_rollback_to_prefix(d["k"], d["v"], d["a"], d["b"], S_in, S_out, kv, n_keep)
            torch.cuda.synchronize()
            assert kv.tolist() == [100 + nk[0], 0 + nk[1], 7 + nk[2]]
            for bb in range(3):
                want = S_in[bb] if nk[bb] == 0 else Sd[nk[bb] - 1][bb]
                assert same_bits(S_out[bb], want), (n, mix, bb)


def test_rollback_oracle_parity_and_clamp():
    T = 9
    r, S0 = _case(700, 2, T, 2, 4, 128, 128)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    _, _, S_T = _verify(d, S_in)
    kv = torch.tensor([5, 6], dtype=torch.int32, device="cuda")
    n_keep = torch.tensor([4, 99], dtype=torch.int32, device="cuda")      # 99 is clamped to T
    S_out = S_T.clone()
    _xv().xv_rollback_to_prefix(d["k"], d["v"], d["a"], d["b"], S_in, S_out, kv, n_keep)
    torch.cuda.synchronize()
    Sn, kv_ref = oracle.rollback(r["k"], r["v"], r["a"], r["b"], S0, np.array([5, 6], np.int32),
                                 np.array([4, 9], np.int32))
    assert kv.tolist() == [9, 15] and kv_ref.tolist() == [9, 15]
    assert rel_l2(S_out.cpu().numpy(), Sn) <= STATE_REL_L2
    assert same_bits(S_out[1], S_T[1])


def test_gdn_batch_invariance():
    """Every request of a batch of 8 gets the bits it gets alone."""
    r, S0 = _case(800, 8, 9, 2, 4, 128, 128)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    o, o32, S = _verify(d, S_in)
    for bb in range(8):
        db = {k: v[bb:bb + 1].contiguous() for k, v in d.items()}
        o1, o321, S1 = _verify(db, S_in[bb:bb + 1].contiguous())
        assert same_bits(o1[0], o[bb]) and same_bits(o321[0], o32[bb]) and same_bits(S1[0], S[bb])


def test_gdn_repeatable():
    r, S0 = _case(900, 2, 9, 2, 6, 128, 128)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    o0, o320, S0d = _verify(d, S_in)
    for _ in range(100):
        o, o32, S = _verify(d, S_in)
        assert same_bits(o32, o320) and same_bits(S, S0d)


def _rows(seed, B, T, Hk, Hv, dk, dv):
    r = random_gdn(np.random.default_rng(seed), B, T, Hk, Hv, dk, dv)
    return _dev(r)


@pytest.mark.parametrize("Tp,T,dk", [(9, 9, 128), (1, 16, 128), (16, 1, 64), (5, 12, 64), (16, 16, 128)])
def test_verify_after_equals_rollback_then_verify(Tp, T, dk):
    """One launch = xv_rollback_to_prefix of the previous call + xv_gdn_verify, bit for bit,
    for every kept count (0, partial, all, and values clamped from outside [0, Tp])."""
    B, Hk, Hv, dv = 6, 2, 4, 64
    prev = _rows(1100 + Tp * 17 + T, B, Tp, Hk, Hv, dk, dv)
    cur = _rows(1200 + Tp * 17 + T, B, T, Hk, Hv, dk, dv)
    S0 = (np.random.default_rng(1300 + T).standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)
    P = torch.from_numpy(S0).cuda()
    _, _, Q = _verify(prev, P)
    nk_list = [0, Tp, min(1, Tp), Tp // 2, -3, Tp + 4]
    nk = torch.tensor(nk_list, dtype=torch.int32, device="cuda")
    # the two-launch reference
    S_roll = Q.clone()
    kv = torch.zeros((B,), dtype=torch.int32, device="cuda")
    _xv().xv_rollback_to_prefix(prev["k"], prev["v"], prev["a"], prev["b"], P, S_roll, kv, nk)
    o_ref, o32_ref, S_ref = _verify(cur, S_roll)
    # one launch
    K, O = torch.full_like(P, float("nan")), torch.full_like(P, float("nan"))
    o = torch.empty_like(o_ref)
    o32 = torch.empty_like(o32_ref)
    P0, Q0 = P.clone(), Q.clone()
    _xv().xv_gdn_verify_after(cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], prev["k"], prev["v"],
                              prev["a"], prev["b"], nk, P, Q, K, O, o, o32)
    torch.cuda.synchronize()
    assert kv.tolist() == [min(max(n, 0), Tp) for n in nk_list]
    assert same_bits(K, S_roll) and same_bits(O, S_ref)
    assert same_bits(o, o_ref) and same_bits(o32, o32_ref)
    assert same_bits(P, P0) and same_bits(Q, Q0)                 # the previous states are read only


def test_verify_after_chain_equals_sequential_decode():
    """Five lazy steps of 9 rows with random kept counts, then the settling rollback:
    every output row that was kept, and the final state, equal one-token decoding of the
    kept rows."""
    B, T, Hk, Hv, dk, dv = 3, 9, 2, 4, 128, 128
    rng = np.random.default_rng(1400)
    S0 = (rng.standard_normal((B, Hv, dk, dv)) * 0.05).astype(np.float32)
    bufs = [torch.from_numpy(S0).cuda()] + [torch.empty((B, Hv, dk, dv), device="cuda") for _ in range(3)]
    P, Q, K, O = bufs
    steps = [_rows(1500 + i, B, T, Hk, Hv, dk, dv) for i in range(5)]
    keeps = [rng.integers(1, T + 1, size=B).astype(np.int32) for _ in steps]
    keeps[2][:] = T                                             # one step that keeps every row
    outs = []
    for i, d in enumerate(steps):
        o = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device="cuda")
        o32 = torch.empty((B, T, Hv, dv), dtype=torch.float32, device="cuda")
        if i == 0:
            _xv().xv_gdn_verify(d["q"], d["k"], d["v"], d["a"], d["b"], P, Q, o, o32)
        else:
            pd, nk = steps[i - 1], torch.from_numpy(keeps[i - 1]).cuda()
            _xv().xv_gdn_verify_after(d["q"], d["k"], d["v"], d["a"], d["b"], pd["k"], pd["v"], pd["a"],
                                      pd["b"], nk, P, Q, K, O, o, o32)
            P, Q, K, O = K, O, P, Q
        outs.append((o, o32))
    kv = torch.zeros((B,), dtype=torch.int32, device="cuda")
    last = steps[-1]
    _xv().xv_rollback_to_prefix(last["k"], last["v"], last["a"], last["b"], P, Q,
                                kv, torch.from_numpy(keeps[-1]).cuda())
    torch.cuda.synchronize()
    for bb in range(B):
        S = torch.from_numpy(S0[bb:bb + 1]).cuda()
        for i, d in enumerate(steps):
            n = int(keeps[i][bb])
            db = {k: v[bb:bb + 1, :n].contiguous() for k, v in d.items()}
            od, o32d, Sd = _decode(db, S, n)
            assert same_bits(outs[i][0][bb, :n], od[0]) and same_bits(outs[i][1][bb, :n], o32d[0]), (bb, i)
            S = Sd[-1]
        assert same_bits(Q[bb], S[0]), bb


@pytest.mark.parametrize("T,dk,dv", [(1, 128, 128), (16, 128, 128), (17, 64, 64), (45, 128, 96), (300, 128, 128)])
def test_gdn_prefill_equals_verify_steps(T, dk, dv):
    """xv_gdn_prefill over T rows gives the outputs and final state of verify steps of at
    most 16 rows (and so of one-token decoding), bit for bit."""
    B, Hk, Hv = 2, 2, 4
    r, S0 = _case(1600 + T + dk, B, T, Hk, Hv, dk, dv)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    S_out = torch.empty_like(S_in)
    o = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((B, T, Hv, dv), dtype=torch.float32, device="cuda")
    _xv().xv_gdn_prefill(d["q"], d["k"], d["v"], d["a"], d["b"], S_in, S_out, o, o32)
    S = S_in.clone()
    o_r, o32_r = torch.empty_like(o), torch.empty_like(o32)
    for t0 in range(0, T, 16):
        tt = min(16, T - t0)
        dt = {k: v[:, t0:t0 + tt].contiguous() for k, v in d.items()}
        os_, o32s, S = _verify(dt, S)
        o_r[:, t0:t0 + tt] = os_; o32_r[:, t0:t0 + tt] = o32s
    torch.cuda.synchronize()
    assert same_bits(o, o_r) and same_bits(o32, o32_r) and same_bits(S_out, S)


@pytest.mark.parametrize("T,dk,dv", [(300, 128, 128), (1000, 64, 64)])
def test_gdn_prefill_vs_oracle(T, dk, dv):
    """xv_gdn_prefill against the fp64 oracle from the same bf16 / fp32 inputs over a long
    prompt: the state within 1e-4 relative L2, the outputs within the output tolerances."""
    B, Hk, Hv = 1, 2, 4
    r, S0 = _case(1700 + T + dk, B, T, Hk, Hv, dk, dv)
    d = _dev(r)
    S_in = torch.from_numpy(S0).cuda()
    S_out = torch.empty_like(S_in)
    o = torch.empty((B, T, Hv, dv), dtype=torch.bfloat16, device="cuda")
    o32 = torch.empty((B, T, Hv, dv), dtype=torch.float32, device="cuda")
    _xv().xv_gdn_prefill(d["q"], d["k"], d["v"], d["a"], d["b"], S_in, S_out, o, o32)
    torch.cuda.synchronize()
    o_ref, S_ref, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    assert rel_l2(S_out.cpu().numpy(), S_ref) <= STATE_REL_L2
    assert max_rel(o32.cpu().numpy(), o_ref) <= OUT_MAX_REL
    assert rel_l2(o32.cpu().numpy(), o_ref) <= OUT_REL_L2
