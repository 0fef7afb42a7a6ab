"""Pins of the fp64 CPU oracle to things other than itself (no GPU needed).

Each check ties an oracle function to an independent fact: brute-force matrix
algebra written from the definition (numpy fp64, explicit d x d products),
exact rational arithmetic, hand-worked examples under tests/golden/, closed
forms and special cases.  They are chosen so that a dropped term, a wrong sign,
a wrong head mapping or a transposed operand in the oracle fails at least one
of them (tests/test_oracle_mutants.py plants such mistakes and checks that).
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_exact_speculative_amd.inputs import (f32_to_bf16_bits, bf16_bits_to_f32,
                                              random_bf16, random_gdn)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *nums = line.split()
            vals[key] = np.array([float(x) for x in nums])
    return vals


def _rel(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(np.ravel(b)), 1e-300)


# ---------------------------------------------------------------------------
# bf16 input helpers (input preparation; pinned so the oracle sees what we think)
# ---------------------------------------------------------------------------
def test_bf16_round_trip_and_ties():
    # exact values survive; ties go to even; nearest otherwise
    x = np.array([1.0, -2.5, 0.0, 3.140625, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9], np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    want = np.array([1.0, -2.5, 0.0, 3.140625, 1.0, 1 + 4 * 2 ** -8, 1.0], np.float32)
    assert np.array_equal(got, want)
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    rb = bf16_bits_to_f32(f32_to_bf16_bits(r))
    assert np.all(np.abs(rb - r) <= np.abs(r) * 2.0 ** -8 + 1e-30)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def test_gemm_matches_numpy_fp64():
    rng = np.random.default_rng(1)
    x = random_bf16(rng, (7, 96))
    w = random_bf16(rng, (48, 96), 0.02)
    y = oracle.gemm(x, w)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64).T
    assert _rel(y, ref) < 1e-14
    # orientation: y[m][n] pairs row m of x with row n of w
    assert abs(y[3, 5] - np.dot(bf16_bits_to_f32(x[3]).astype(np.float64),
                                bf16_bits_to_f32(w[5]).astype(np.float64))) < 1e-12


def test_gemm_exact_integers():
    """Integer-valued x and w/64: every partial sum is exact, so y is exact."""
    rng = np.random.default_rng(2)
    xi = rng.integers(-4, 5, size=(5, 256))
    wi = rng.integers(-4, 5, size=(40, 256))
    x = f32_to_bf16_bits(xi.astype(np.float32))
    w = f32_to_bf16_bits((wi / 64.0).astype(np.float32))
    y = oracle.gemm(x, w)
    exact = (xi @ wi.T) / 64.0
    assert np.array_equal(y, exact)


# ---------------------------------------------------------------------------
# GDN: brute force with explicit (I - b k k^T)
# ---------------------------------------------------------------------------
def _gdn_brute(q, k, v, a, b, S0):
    """Literal S_t = a S (I - b k k^T) + b v k^T, o_t = S_t q_t with d x d products.

    Layout conversions are explicit: S0 is stored [B][Hv][dk][dv] (element
    (j, i) of the d_v x d_k matrix at [i][j]); the key head of value head h is
    h // (Hv // Hk) (each key head serves a contiguous group of value heads).
    """
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    qf = bf16_bits_to_f32(q).astype(np.float64)
    kf = bf16_bits_to_f32(k).astype(np.float64)
    vf = bf16_bits_to_f32(v).astype(np.float64)
    grp = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    Sall = np.zeros((B, T + 1, Hv, dk, dv))
    for bb in range(B):
        for h in range(Hv):
            g = h // grp
            S = S0[bb, h].astype(np.float64).T.copy()     # d_v x d_k
            Sall[bb, 0, h] = S.T
            for t in range(T):
                kt = kf[bb, t, g]
                At = np.eye(dk) - float(b[bb, t, h]) * np.outer(kt, kt)
                S = float(a[bb, t, h]) * (S @ At) + float(b[bb, t, h]) * np.outer(vf[bb, t, h], kt)
                o[bb, t, h] = S @ qf[bb, t, g]
                Sall[bb, t + 1, h] = S.T
    return o, Sall


@pytest.mark.parametrize("shape", [(1, 5, 2, 4, 16, 16), (2, 3, 1, 3, 8, 12), (1, 9, 2, 4, 64, 64)])
def test_gdn_matches_brute_force(shape):
    B, T, Hk, Hv, dk, dv = shape
    rng = np.random.default_rng(3)
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32) * np.float32(0.1)
    o, ST, Sall = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0, want_all=True)
    ob, Sb = _gdn_brute(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    assert _rel(o, ob) < 1e-12
    assert _rel(Sall, Sb) < 1e-12
    assert _rel(ST, Sb[:, -1]) < 1e-12
    assert np.array_equal(Sall[:, 0], S0.astype(np.float64))


def test_gdn_exact_rationals():
    """dk = dv = 4, T = 3 in exact rational arithmetic (bf16/fp32 inputs are dyadic)."""
    rng = np.random.default_rng(4)
    B, T, Hk, Hv, dk, dv = 1, 3, 1, 2, 4, 4
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = (rng.standard_normal((B, Hv, dk, dv)) * 0.5).astype(np.float32)
    o, ST, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    qf = bf16_bits_to_f32(r["q"]); kf = bf16_bits_to_f32(r["k"]); vf = bf16_bits_to_f32(r["v"])
    for h in range(Hv):
        g = h // (Hv // Hk)
        S = [[Fraction(float(S0[0, h, i, j])) for i in range(dk)] for j in range(dv)]
        for t in range(T):
            a = Fraction(float(r["a"][0, t, h])); b = Fraction(float(r["b"][0, t, h]))
            kk = [Fraction(float(x)) for x in kf[0, t, g]]
            qq = [Fraction(float(x)) for x in qf[0, t, g]]
            vv = [Fraction(float(x)) for x in vf[0, t, h]]
            A = [[(1 if i == c else 0) - b * kk[i] * kk[c] for c in range(dk)] for i in range(dk)]
            P = [[sum(S[j][l] * A[l][c] for l in range(dk)) for c in range(dk)] for j in range(dv)]
            S = [[a * P[j][c] + b * vv[j] * kk[c] for c in range(dk)] for j in range(dv)]
            for j in range(dv):
                ex = sum(S[j][c] * qq[c] for c in range(dk))
                assert abs(o[0, t, h, j] - float(ex)) <= 1e-15 * max(1.0, abs(float(ex)))
        for j in range(dv):
            for i in range(dk):
                assert abs(ST[0, h, i, j] - float(S[j][i])) <= 1e-15 * max(1.0, abs(float(S[j][i])))


def test_gdn_hand_worked_golden():
    gv = _golden("gdn_hand_2x2.txt")
    q = np.zeros((1, 2, 1, 2), np.uint16); k = np.zeros_like(q); v = np.zeros((1, 2, 1, 2), np.uint16)
    for t in range(2):
        q[0, t, 0] = f32_to_bf16_bits(gv["q%d" % (t + 1)].astype(np.float32))
        k[0, t, 0] = f32_to_bf16_bits(gv["k%d" % (t + 1)].astype(np.float32))
        v[0, t, 0] = f32_to_bf16_bits(gv["v%d" % (t + 1)].astype(np.float32))
    a = gv["a"].astype(np.float32).reshape(1, 2, 1)
    b = gv["b"].astype(np.float32).reshape(1, 2, 1)
    S0m = gv["S0"].reshape(2, 2)                                  # (j, i)
    S0 = S0m.T.astype(np.float32).reshape(1, 1, 2, 2)             # stored [i][j]
    o, ST, Sall = oracle.gdn(q, k, v, a, b, S0, want_all=True)
    assert np.array_equal(o[0, 0, 0], gv["o1"])
    assert np.array_equal(o[0, 1, 0], gv["o2"])
    assert np.array_equal(Sall[0, 1, 0].T.ravel(), gv["S1"])
    assert np.array_equal(ST[0, 0].T.ravel(), gv["S2"])


def _unit_rows(Hk, dk, idx):
    k = np.zeros((Hk, dk), np.float32)
    k[:, idx] = 1.0
    return f32_to_bf16_bits(k)


def test_gdn_special_beta_zero_is_pure_decay():
    rng = np.random.default_rng(5)
    B, T, Hk, Hv, dk, dv = 1, 6, 2, 4, 8, 8
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    bz = np.zeros_like(r["b"])
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    o, ST, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], bz, S0)
    qf = bf16_bits_to_f32(r["q"]).astype(np.float64)
    for h in range(Hv):
        g = h // 2
        prod = 1.0
        for t in range(T):
            prod *= float(r["a"][0, t, h])
            want = prod * (S0[0, h].astype(np.float64).T @ qf[0, t, g])
            assert np.allclose(o[0, t, h], want, rtol=1e-12, atol=1e-14)
        assert np.allclose(ST[0, h], prod * S0[0, h].astype(np.float64), rtol=1e-12, atol=1e-14)


def test_gdn_special_unit_key_full_write():
    """a = b = 1 and k a unit basis vector: the new state maps k exactly to v."""
    rng = np.random.default_rng(6)
    B, T, Hk, Hv, dk, dv = 1, 4, 1, 2, 8, 6
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    for t in range(T):
        r["k"][0, t] = _unit_rows(Hk, dk, (3 * t + 1) % dk)
    ones = np.ones_like(r["a"])
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    _, _, Sall = oracle.gdn(r["q"], r["k"], r["v"], ones, ones, S0, want_all=True)
    vf = bf16_bits_to_f32(r["v"]).astype(np.float64)
    for t in range(T):
        idx = (3 * t + 1) % dk
        for h in range(Hv):
            S = Sall[0, t + 1, h].T                       # d_v x d_k
            assert np.allclose(S[:, idx], vf[0, t, h], rtol=0, atol=1e-14)


def test_gdn_special_zero_state_single_token():
    rng = np.random.default_rng(7)
    B, T, Hk, Hv, dk, dv = 1, 1, 2, 6, 16, 8
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = np.zeros((B, Hv, dk, dv), np.float32)
    o, _, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    qf = bf16_bits_to_f32(r["q"]).astype(np.float64)
    kf = bf16_bits_to_f32(r["k"]).astype(np.float64)
    vf = bf16_bits_to_f32(r["v"]).astype(np.float64)
    for h in range(Hv):
        g = h // 3
        want = float(r["b"][0, 0, h]) * np.dot(kf[0, 0, g], qf[0, 0, g]) * vf[0, 0, h]
        assert np.allclose(o[0, 0, h], want, rtol=1e-13, atol=1e-15)


def test_gdn_special_repeated_key_is_ema():
    """Same unit key every step and a = 1: S_t k = (1 - b) S_{t-1} k + b v (moving average)."""
    rng = np.random.default_rng(8)
    B, T, Hk, Hv, dk, dv = 1, 7, 1, 1, 4, 5
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    for t in range(T):
        r["k"][0, t] = _unit_rows(Hk, dk, 2)
    ones = np.ones_like(r["a"])
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    _, _, Sall = oracle.gdn(r["q"], r["k"], r["v"], ones, r["b"], S0, want_all=True)
    vf = bf16_bits_to_f32(r["v"]).astype(np.float64)
    m = S0[0, 0, 2].astype(np.float64)        # S_0 k = row i=2 of the stored layout
    for t in range(T):
        bt = float(r["b"][0, t, 0])
        m = (1 - bt) * m + bt * vf[0, t, 0]
        assert np.allclose(Sall[0, t + 1, 0, 2], m, rtol=1e-13, atol=1e-15)


def test_gdn_head_mapping_and_batch_independence():
    rng = np.random.default_rng(9)
    B, T, Hk, Hv, dk, dv = 3, 4, 2, 6, 8, 8
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    o, ST, _ = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0)
    for bb in range(B):
        sl = slice(bb, bb + 1)
        o1, S1, _ = oracle.gdn(r["q"][sl], r["k"][sl], r["v"][sl], r["a"][sl], r["b"][sl], S0[sl])
        assert np.array_equal(o1[0], o[bb]) and np.array_equal(S1[0], ST[bb])
    # value heads 0..2 use key head 0, 3..5 key head 1: swapping key heads swaps groups
    q2 = r["q"][:, :, ::-1].copy(); k2 = r["k"][:, :, ::-1].copy()
    perm = [3, 4, 5, 0, 1, 2]
    o2, _, _ = oracle.gdn(q2, k2, r["v"][:, :, perm].copy(), r["a"][:, :, perm].copy(),
                          r["b"][:, :, perm].copy(), S0[:, perm].copy())
    assert np.array_equal(o2[:, :, perm], o)


def test_rollback_oracle():
    rng = np.random.default_rng(10)
    B, T, Hk, Hv, dk, dv = 3, 5, 1, 2, 8, 8
    r = random_gdn(rng, B, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((B, Hv, dk, dv)).astype(np.float32)
    _, _, Sall = oracle.gdn(r["q"], r["k"], r["v"], r["a"], r["b"], S0, want_all=True)
    kv = np.array([10, 0, 7], np.int32)
    n = np.array([0, 5, 2], np.int32)
    Sn, kv2 = oracle.rollback(r["k"], r["v"], r["a"], r["b"], S0, kv, n)
    assert np.array_equal(kv2, kv + n)
    for bb in range(B):
        assert np.array_equal(Sn[bb], Sall[bb, n[bb]])
    assert np.array_equal(Sn[0], S0[0].astype(np.float64))


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _attn_brute(q, k_new, v_new, k_cache, v_cache, L0, scale):
    """softmax(Q K^T * scale + causal mask) V over [cache | new rows], per (b, kv head)."""
    B, T, Hq, d = q.shape
    Hkv = k_new.shape[2]
    grp = Hq // Hkv
    o = np.zeros((B, T, Hq, d))
    for bb in range(B):
        n = int(L0[bb])
        for g in range(Hkv):
            K = np.concatenate([bf16_bits_to_f32(k_cache[bb, g, :n]),
                                bf16_bits_to_f32(k_new[bb, :, g])]).astype(np.float64)
            V = np.concatenate([bf16_bits_to_f32(v_cache[bb, g, :n]),
                                bf16_bits_to_f32(v_new[bb, :, g])]).astype(np.float64)
            for hh in range(grp):
                h = g * grp + hh
                Q = bf16_bits_to_f32(q[bb, :, h]).astype(np.float64)     # T x d
                S = scale * (Q @ K.T)                                      # T x (n+T)
                mask = np.arange(n + T)[None, :] > (n + np.arange(T))[:, None]
                S[mask] = -np.inf
                S = S - S.max(axis=1, keepdims=True)
                P = np.exp(S)
                P /= P.sum(axis=1, keepdims=True)
                o[bb, :, h] = P @ V
    return o


def _attn_case(rng, B, T, Hq, Hkv, d, L0, Lmax, poison=True):
    q = random_bf16(rng, (B, T, Hq, d))
    kn = random_bf16(rng, (B, T, Hkv, d)); vn = random_bf16(rng, (B, T, Hkv, d))
    fill = 0x7FC0 if poison else 0
    kc = np.full((B, Hkv, Lmax, d), fill, np.uint16); vc = np.full_like(kc, fill)
    for bb in range(B):
        kc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
        vc[bb, :, :L0[bb]] = random_bf16(rng, (Hkv, L0[bb], d))
    return q, kn, vn, kc, vc, np.asarray(L0, np.int32)


@pytest.mark.parametrize("cfg", [(1, 5, 4, 1, 64, [128]), (2, 3, 6, 2, 32, [0, 17]), (3, 9, 6, 3, 16, [1, 40, 5])])
def test_attn_matches_brute_force(cfg):
    B, T, Hq, Hkv, d, L0 = cfg
    rng = np.random.default_rng(11)
    Lmax = max(L0) + T + 3
    q, kn, vn, kc, vc, L0 = _attn_case(rng, B, T, Hq, Hkv, d, L0, Lmax)
    scale = 1.0 / np.sqrt(d)
    o = oracle.attn(q, kn, vn, kc, vc, L0, scale)
    ob = _attn_brute(q, kn, vn, kc, vc, L0, scale)
    assert np.all(np.isfinite(o))             # never reads a poisoned slot
    assert _rel(o, ob) < 1e-12
    for (bb, r, h) in [(0, 0, 0), (B - 1, T - 1, Hq - 1), (0, T // 2, Hq // 2)]:
        assert np.array_equal(oracle.attn_row(q, kn, vn, kc, vc, L0, scale, bb, r, h), o[bb, r, h])


def test_attn_hand_worked_golden():
    gv = _golden("attn_hand_d2.txt")
    kc = np.full((1, 1, 6, 2), 0x7FC0, np.uint16); vc = kc.copy()
    kc[0, 0, :2] = f32_to_bf16_bits(gv["kc"].astype(np.float32).reshape(2, 2))
    vc[0, 0, :2] = f32_to_bf16_bits(gv["vc"].astype(np.float32).reshape(2, 2))
    kn = f32_to_bf16_bits(gv["kn"].astype(np.float32).reshape(1, 2, 1, 2))
    vn = f32_to_bf16_bits(gv["vn"].astype(np.float32).reshape(1, 2, 1, 2))
    q = f32_to_bf16_bits(gv["q"].astype(np.float32).reshape(1, 2, 1, 2))
    o = oracle.attn(q, kn, vn, kc, vc, np.array([2], np.int32), 1.0)
    assert np.allclose(o[0, 0, 0], gv["o0"], rtol=0, atol=1e-14)
    assert np.allclose(o[0, 1, 0], gv["o1"], rtol=0, atol=1e-14)


def test_attn_special_cases():
    rng = np.random.default_rng(12)
    d = 32
    # length 1: the only visible value
    q, kn, vn, kc, vc, L0 = _attn_case(rng, 1, 1, 2, 1, d, [0], 4)
    o = oracle.attn(q, kn, vn, kc, vc, L0, 0.125)
    for h in range(2):
        assert np.array_equal(o[0, 0, h], bf16_bits_to_f32(vn[0, 0, 0]).astype(np.float64))
    # identical keys: the plain mean of the visible values
    q, kn, vn, kc, vc, L0 = _attn_case(rng, 1, 3, 2, 1, d, [20], 30)
    key = random_bf16(rng, (d,))
    kc[0, 0, :20] = key; kn[0, :, 0] = key
    o = oracle.attn(q, kn, vn, kc, vc, L0, 0.125)
    V = np.concatenate([bf16_bits_to_f32(vc[0, 0, :20]), bf16_bits_to_f32(vn[0, :, 0])]).astype(np.float64)
    for r in range(3):
        assert np.allclose(o[0, r, 0], V[:21 + r].mean(axis=0), rtol=1e-12, atol=1e-13)
    # one dominant key (score margin ~60): its value
    q, kn, vn, kc, vc, L0 = _attn_case(rng, 1, 1, 1, 1, d, [10], 12)
    qv = np.zeros(d, np.float32); qv[0] = 1.0
    q[0, 0, 0] = f32_to_bf16_bits(qv)
    kk = np.zeros((10, d), np.float32); kk[4, 0] = 60.0
    kc[0, 0, :10] = f32_to_bf16_bits(kk)
    kn[0, 0, 0] = f32_to_bf16_bits(np.zeros(d, np.float32))
    o = oracle.attn(q, kn, vn, kc, vc, L0, 1.0)
    assert np.allclose(o[0, 0, 0], bf16_bits_to_f32(vc[0, 0, 4]), rtol=1e-15, atol=1e-15)


def test_attn_causality_and_capacity():
    rng = np.random.default_rng(13)
    q, kn, vn, kc, vc, L0 = _attn_case(rng, 1, 6, 4, 2, 16, [33], 40)
    o = oracle.attn(q, kn, vn, kc, vc, L0, 0.25)
    # row r must not see new rows > r
    kn2 = kn.copy(); vn2 = vn.copy()
    kn2[0, 4:] = random_bf16(rng, kn2[0, 4:].shape); vn2[0, 4:] = random_bf16(rng, vn2[0, 4:].shape)
    o2 = oracle.attn(q, kn2, vn2, kc, vc, L0, 0.25)
    assert np.array_equal(o[0, :4], o2[0, :4]) and not np.array_equal(o[0, 4:], o2[0, 4:])
    # a larger capacity with other padding changes nothing
    kc3 = np.zeros((1, 2, 400, 16), np.uint16); vc3 = np.zeros_like(kc3)
    kc3[:, :, :40] = kc; vc3[:, :, :40] = vc
    o3 = oracle.attn(q, kn, vn, kc3, vc3, L0, 0.25)
    assert np.array_equal(o, o3)


# ---------------------------------------------------------------------------
# Greedy acceptance
# ---------------------------------------------------------------------------
def test_greedy_ties_and_acceptance():
    logits = np.zeros((2, 4, 6))
    logits[0, 0, [2, 5]] = 3.0          # tie -> 2
    logits[0, 1, 4] = 1.0
    logits[0, 2, 0] = -1.0               # all others 0 -> lowest index among zeros is 1
    logits[0, 3, 3] = 2.0
    logits[1, :, 1] = 1.0
    draft = np.array([[9, 2, 4, 7], [0, 1, 1, 1]], np.int32)
    ids, n = oracle.greedy(logits, draft)
    assert ids.tolist() == [[2, 4, 1, 3], [1, 1, 1, 1]]
    assert n.tolist() == [3, 4]
    # brute force over random small cases
    rng = np.random.default_rng(14)
    for _ in range(200):
        B, T, N = 2, int(rng.integers(1, 6)), int(rng.integers(1, 5))
        lg = rng.integers(0, 3, size=(B, T, N)).astype(np.float64)
        dr = rng.integers(0, N, size=(B, T)).astype(np.int32)
        ids, n = oracle.greedy(lg, dr)
        for bb in range(B):
            want_ids = [int(np.flatnonzero(lg[bb, t] == lg[bb, t].max())[0]) for t in range(T)]
            assert ids[bb].tolist() == want_ids
            acc = 0
            for t in range(T - 1):
                if dr[bb, t + 1] != want_ids[t]:
                    break
                acc += 1
            assert n[bb] == acc + 1


# ---------------------------------------------------------------------------
# Logprob of the chosen token (log-softmax at an index)
# ---------------------------------------------------------------------------
def test_logprob_closed_forms():
    N = 37
    # equal logits (not zero, so that a missing max shift shows): every index has -ln N
    z = np.full((1, 2, N), 3.25)
    ids = np.array([[0, 17]], np.int32)
    assert np.allclose(oracle.logprob(z, ids), -np.log(N), rtol=0, atol=1e-14)
    # one logit raised by D over the rest: closed forms at the raised index and elsewhere
    D = 2.5
    z = np.full((1, 2, N), -1.0)
    z[0, :, 5] += D
    lp = oracle.logprob(z, np.array([[5, 9]], np.int32))
    top = -np.log1p((N - 1) * np.exp(-D))
    assert abs(lp[0, 0] - top) < 1e-14 and abs(lp[0, 1] - (top - D)) < 1e-14


def test_logprob_normalises_and_is_shift_invariant():
    rng = np.random.default_rng(3)
    B, T, N = 2, 3, 50
    z = rng.standard_normal((B, T, N)) * 4.0
    full = np.stack([oracle.logprob(z, np.full((B, T), n, np.int32)) for n in range(N)], axis=-1)
    assert np.allclose(np.exp(full).sum(-1), 1.0, rtol=0, atol=1e-13)
    # the differences between indices are the logit differences
    assert np.allclose(full - full[..., :1], z - z[..., :1], rtol=0, atol=1e-12)
    shifted = np.stack([oracle.logprob(z + 100.0, np.full((B, T), n, np.int32)) for n in range(N)], axis=-1)
    assert np.allclose(shifted, full, rtol=0, atol=1e-12)
    # each row is its own: permuting the rows permutes the results
    zp = z[::-1].copy()
    assert np.array_equal(oracle.logprob(zp, np.full((B, T), 7, np.int32)),
                          oracle.logprob(z, np.full((B, T), 7, np.int32))[::-1])
