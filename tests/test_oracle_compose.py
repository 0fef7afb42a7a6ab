"""Pins of the composed-decoding oracle (oracle/compose.py); CPU only.

round_bf16 against a brute-force search of the bf16 grid; the per-head split
against hand indexing and closed forms; and the property the post reports,
checked on the oracle itself: greedy decoding with speculative verification
emits the same ids, logprobs, GDN state and KV cache as decoding without it,
whatever the drafts.
"""
import numpy as np
import pytest

import oracle
from oracle import compose as C
from bit_exact_speculative_amd import inputs as gen


def _bf16_brute(x: float) -> int:
    """Nearest bf16 bit pattern by scanning the neighbours of the truncated pattern."""
    u = int(np.array([x], np.float32).view(np.uint32)[0]) >> 16       # within 1 ulp of x
    best = None
    for h in range(max(u - 2, 0), u + 3):
        if (h & 0x7F80) == 0x7F80:
            continue
        v = float((np.array([h], np.uint32) << 16).view(np.float32)[0])
        key = (abs(v - x), h & 1)                                    # nearer, then even
        if best is None or key < best[0]:
            best = (key, h)
    return best[1]


def test_round_bf16_matches_brute_force():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000),
                         [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 2.0 - 2 ** -9,
                          0.5, 3.0 * 2 ** -7]])
    xs = np.concatenate([xs, -xs])
    got = C.round_bf16(xs)
    want = np.array([_bf16_brute(abs(float(x))) | (0x8000 if x < 0 else 0) for x in xs], np.uint16)
    assert np.array_equal(got, want)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 and goes to the even 1.0
    assert C.round_bf16(np.array([1 + 2 ** -8]))[0] == 0x3F80
    assert C.round_bf16(np.array([1 + 3 * 2 ** -8]))[0] == 0x3F82


def _shapes():
    return C.Shapes(Hk=2, Hv=4, dk=8, dv=8, Hq=4, Hkv=2, d=16)


def test_split_columns_and_closed_forms():
    s = _shapes()
    rng = np.random.default_rng(1)
    M = 3
    N1 = 2 * s.Hk * s.dk + s.Hv * s.dv
    N2 = s.Hq * s.d + 2 * s.Hkv * s.d + 2 * s.Hv + 5
    y1 = gen.random_bf16(rng, (M, N1))
    y2 = gen.random_bf16(rng, (M, N2))
    # beta logits = -decay logits, and one zero of each
    off = s.Hq * s.d + 2 * s.Hkv * s.d
    y2[:, off + s.Hv:off + 2 * s.Hv] = y2[:, off:off + s.Hv] ^ np.uint16(0x8000)
    y2[0, off] = 0
    y2[0, off + s.Hv] = 0
    sp = C.split(y1, y2, s)
    val = C.bf16_value
    for m in range(M):
        for h in range(s.Hk):
            for name, base in (("q", 0), ("k", s.Hk * s.dk)):
                u = val(y1[m, base + h * s.dk: base + (h + 1) * s.dk])
                got = sp[name][m, h]
                # unit norm up to the epsilon, and the direction of u
                assert abs(np.linalg.norm(got) - np.sqrt(u @ u / (u @ u + C.L2_EPS))) < 1e-14
                assert np.allclose(got * np.linalg.norm(u), u * np.linalg.norm(got), rtol=0, atol=1e-13)
        for h in range(s.Hv):
            for j in range(s.dv):
                assert sp["v"][m, h, j] == y1[m, 2 * s.Hk * s.dk + h * s.dv + j]
        for h in range(s.Hq):
            for j in range(s.d):
                assert sp["q_attn"][m, h, j] == y2[m, h * s.d + j]
        for g in range(s.Hkv):
            for j in range(s.d):
                assert sp["k_new"][m, g, j] == y2[m, s.Hq * s.d + g * s.d + j]
                assert sp["v_new"][m, g, j] == y2[m, s.Hq * s.d + s.Hkv * s.d + g * s.d + j]
    # decay = exp(-softplus(alpha)) and beta = sigmoid(beta logit): with beta logit = -alpha
    # the two are the same number, a half at zero
    alpha = val(y2[:, off:off + s.Hv])
    assert np.allclose(sp["a"], np.exp(-np.logaddexp(0.0, alpha)), rtol=1e-15, atol=0)
    assert np.allclose(sp["a"], sp["b"], rtol=1e-15, atol=0)
    assert sp["a"][0, 0] == 0.5 and sp["b"][0, 0] == 0.5


def _tiny_model(Lextra=64):
    wl = gen.WORKLOADS["tiny"]
    inp = gen.composed_inputs(wl, Lmax=wl.L0 + Lextra)
    s = C.Shapes(wl.Hk, wl.Hv, wl.dk, wl.dv, wl.Hq, wl.Hkv, wl.d)
    m = C.Model(inp.extra["E"], inp.W1, inp.W2, inp.Wh_gdn, inp.Wh_attn, s)
    p = inp.prefix
    _, S, _ = oracle.gdn(p["q"], p["k"], p["v"], p["a"], p["b"],
                         np.zeros((wl.B, wl.Hv, wl.dk, wl.dv), np.float32))
    st = C.State(S.astype(np.float32), inp.k_cache.copy(), inp.v_cache.copy(), inp.L0.copy())
    return m, st, inp.extra["root"], wl


@pytest.mark.parametrize("k,p_wrong", [(1, 0.0), (4, 0.3), (8, 0.5), (8, 1.0)])
def test_speculative_decoding_equals_plain_decoding_in_the_oracle(k, p_wrong):
    m, st0, root, wl = _tiny_model()
    n = 14
    st_a = st0.copy()
    ids_a, lp_a, keeps_a, _ = C.generate(m, st_a, root, n)
    assert all(int(x[0]) == 1 for x in keeps_a)
    rng = np.random.default_rng(k * 10 + int(p_wrong * 10))

    def drafts(b, pos, kk):
        d = np.array([ids_a[b, min(pos + i, n - 1)] for i in range(kk)], np.int32)
        bad = rng.random(kk) < p_wrong
        d[bad] = (d[bad] + 1 + rng.integers(0, wl.NH - 1, int(bad.sum()))) % wl.NH
        return d

    st_b = st0.copy()
    ids_b, lp_b, keeps_b, _ = C.generate(m, st_b, root, n, drafts, k=k)
    assert np.array_equal(ids_a, ids_b) and np.array_equal(lp_a, lp_b)
    if p_wrong == 1.0:
        assert all(int(x[0]) == 1 for x in keeps_b)          # every draft rejected
    elif p_wrong == 0.0:
        assert max(int(x[0]) for x in keeps_b) == k + 1       # all drafts of a step accepted
    # the end states agree once both have consumed the same tokens: the speculative loop
    # may overshoot n in its last step, so plain decoding is rerun to its length
    emitted = int(st_b.kv_len[0] - st0.kv_len[0])
    assert emitted >= n
    st_c = st0.copy()
    C.generate(m, st_c, root, emitted)
    assert np.array_equal(st_c.kv_len, st_b.kv_len) and np.array_equal(st_c.S, st_b.S)
    assert np.array_equal(st_c.kc, st_b.kc) and np.array_equal(st_c.vc, st_b.vc)


def test_step_rows_are_independent_of_the_other_rows():
    """A step's row r gives the bits of the same row in a shorter step (the oracle's
    arithmetic per row does not depend on T)."""
    m, st0, root, wl = _tiny_model()
    toks = np.array([[int(root[0]), 3, 77, 501, 9]], np.int32)
    ids, lp, _, logits = C.step(m, st0.copy(), toks)
    for T in (1, 2, 4):
        ids2, lp2, _, logits2 = C.step(m, st0.copy(), toks[:, :T].copy())
        assert np.array_equal(logits2, logits[:, :T]) and np.array_equal(ids2, ids[:, :T])
        assert np.array_equal(lp2, lp[:, :T])


def test_prefill_equals_forced_one_token_steps_in_the_oracle():
    """The oracle's prefill (every prompt row kept) leaves the state, cache and length of
    feeding the prompt one token at a time, and its last row's logits, id and logprob are
    those of the last one-token step; splitting the prompt in two changes nothing."""
    m, st0, root, wl = _tiny_model()
    rng = np.random.default_rng(21)
    P = 11
    prompt = rng.integers(0, wl.NH, size=(wl.B, P)).astype(np.int32)
    st_a = st0.copy()
    id_a, lp_a, z_a = C.prefill(m, st_a, prompt)
    st_b = st0.copy()
    for t in range(P):
        ids, lp, n_keep, z = C.step(m, st_b, prompt[:, t:t + 1].copy())
        assert np.all(n_keep == 1)
    assert np.array_equal(z[:, 0], z_a) and np.array_equal(ids[:, 0], id_a) and np.array_equal(lp[:, 0], lp_a)
    assert np.array_equal(st_a.S, st_b.S) and np.array_equal(st_a.kv_len, st_b.kv_len)
    assert np.array_equal(st_a.kc, st_b.kc) and np.array_equal(st_a.vc, st_b.vc)
    assert np.all(st_a.kv_len == st0.kv_len + P)
    st_c = st0.copy()
    C.prefill(m, st_c, prompt[:, :4].copy())
    id_c, lp_c, z_c = C.prefill(m, st_c, prompt[:, 4:].copy())
    assert np.array_equal(z_c, z_a) and np.array_equal(st_c.S, st_a.S) and np.array_equal(st_c.kc, st_a.kc)
    # the first generated token is the argmax of the last row (lowest index on ties)
    assert np.array_equal(id_a, np.argmax(z_a, axis=-1))
