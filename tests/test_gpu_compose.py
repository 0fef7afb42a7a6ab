"""Composed decoding on the GPU: the embedding gather and the projection split
against the oracle, the logprob of the greedy id against the oracle, and greedy
decoding with speculative verification against decoding without it (bit for
bit) and against the oracle's composed decoding."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compose as OC
from bit_exact_speculative_amd import inputs as gen
from tests.gpu_util import same_bits, prefix_state

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _host16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,V,H", [(9, 4096, 5120), (1, 512, 256), (72, 4096, 5120), (3, 7, 8)])
def test_embed_rows_is_a_gather(M, V, H):
    rng = np.random.default_rng(M + V)
    E = gen.random_bf16(rng, (V, H))
    tok = rng.integers(0, V, size=M).astype(np.int32)
    x = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    _xv().xv_embed_rows(_dev16(E), torch.from_numpy(tok).cuda(), x)
    torch.cuda.synchronize()
    assert np.array_equal(_host16(x), E[tok])


SPLIT_CASES = [  # M, Hk, Hv, dk, dv, Hq, Hkv, d, extra columns of y1 / y2
    (9, 16, 48, 128, 128, 24, 4, 256, 0, 9120),
    (5, 2, 4, 64, 64, 4, 1, 64, 0, 120),
    (3, 3, 6, 128, 32, 6, 2, 128, 16, 12),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[str(c) for c in SPLIT_CASES])
def test_split_projections_vs_oracle(case):
    M, Hk, Hv, dk, dv, Hq, Hkv, d, x1, x2 = case
    s = OC.Shapes(Hk, Hv, dk, dv, Hq, Hkv, d)
    N1 = 2 * Hk * dk + Hv * dv + x1
    N2 = Hq * d + 2 * Hkv * d + 2 * Hv + x2
    rng = np.random.default_rng(M * 7 + Hk)
    y1 = gen.random_bf16(rng, (M, N1), 1.4)
    y2 = gen.random_bf16(rng, (M, N2), 1.4)
    y1[0, :dk] = 0                                   # an all-zero head: the epsilon keeps it finite
    ref = OC.split(y1, y2, s)
    e = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device="cuda")
    f = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    q, k, v = e(M, Hk, dk), e(M, Hk, dk), e(M, Hv, dv)
    a, b = f(M, Hv), f(M, Hv)
    qa, kn, vn = e(M, Hq, d), e(M, Hkv, d), e(M, Hkv, d)
    _xv().xv_split_projections(_dev16(y1), _dev16(y2), q, k, v, a, b, qa, kn, vn)
    torch.cuda.synchronize()
    # q, k: fp32 normalisation then one bf16 rounding: within half a bf16 ulp (at most 2^-8
    # of the value) plus the fp32 error of a 12-deep sum, a square root, a division and a
    # product (< 2^-16 relative); an all-zero head stays exactly zero
    for name, got in (("q", q), ("k", k)):
        g = OC.bf16_value(_host16(got))
        r = ref[name]
        assert np.all(np.abs(g - r) <= (2.0 ** -8 + 2.0 ** -16) * np.abs(r)), name
    assert not np.any(OC.bf16_value(_host16(q))[0, 0])
    for name, got in (("v", v), ("q_attn", qa), ("k_new", kn), ("v_new", vn)):
        assert np.array_equal(_host16(got), ref[name]), name
    # decay and beta: an exp, an add and a division in fp32
    for name, got in (("a", a), ("b", b)):
        g = got.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - ref[name]) <= 2.0 ** -20 * ref[name]), name


def test_split_rows_do_not_depend_on_the_row_count():
    M, Hk, Hv, dk, dv, Hq, Hkv, d = 12, 16, 48, 128, 128, 24, 4, 256
    rng = np.random.default_rng(11)
    y1 = gen.random_bf16(rng, (M, 2 * Hk * dk + Hv * dv))
    y2 = gen.random_bf16(rng, (M, Hq * d + 2 * Hkv * d + 2 * Hv + 8))
    outs = []
    for rows in (slice(0, M), slice(5, 6)):
        m = rows.stop - rows.start
        e = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device="cuda")
        f = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
        o = [e(m, Hk, dk), e(m, Hk, dk), e(m, Hv, dv), f(m, Hv), f(m, Hv), e(m, Hq, d), e(m, Hkv, d), e(m, Hkv, d)]
        _xv().xv_split_projections(_dev16(y1[rows]), _dev16(y2[rows]), *o)
        outs.append(o)
    torch.cuda.synchronize()
    for big, one in zip(outs[0], outs[1]):
        assert same_bits(big[5:6], one)


def _logprob_bound(N: int, lp: np.ndarray) -> np.ndarray:
    """|lp_gpu - lp_exact| for fp32 logits.  Along the kernel's path to S a value passes
    a 16-column block (one exp2 with the rounding of a subtraction and a product in its
    argument, four additions: under 8 units of 2^-24) and then up to ceil(N / 4096)
    chain folds, six butterfly levels and three wave folds, each a rescaling by an
    exp2 and a product and one addition (under 18 units); the log2 and the ln 2 product
    add 2^-22 |lp|, and 2^-20 covers the exp2 of the largest arguments."""
    depth = 8 + 18 * (-(-N // 4096) + 9)
    return depth * 2.0 ** -24 + 2.0 ** -22 * np.abs(lp) + 2.0 ** -20


@pytest.mark.parametrize("B,T,N", [(1, 9, 4096), (8, 9, 4096), (2, 16, 1000), (1, 5, 7), (1, 1, 12289)])
def test_logprob_vs_oracle_and_invariance(B, T, N):
    xv = _xv()
    rng = np.random.default_rng(B * 100 + N)
    la = (rng.standard_normal((B, T, N)) * 3).astype(np.float32)
    lb = (rng.standard_normal((B, T, N)) * 0.5).astype(np.float32)
    z = (la + lb).astype(np.float64)                 # the same fp32 sum the kernel forms
    dla, dlb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
    draft = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    ids = torch.empty((B, T), dtype=torch.int32, device="cuda")
    nk = torch.empty((B,), dtype=torch.int32, device="cuda")
    lp = torch.empty((B, T), dtype=torch.float32, device="cuda")
    xv.xv_greedy_accept(dla, dlb, draft, ids, nk, lp)
    torch.cuda.synchronize()
    ids_ref, _ = oracle.greedy(z, np.zeros((B, T), np.int32))
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    ref = oracle.logprob(z, ids_ref)
    g = lp.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(g - ref) <= _logprob_bound(N, ref))
    # one row alone, and through the 4-byte-load path (a view 4 bytes into its buffer),
    # gives the same bits
    bb, tt = B - 1, T - 1
    for off in (0, 1):
        buf_a = torch.zeros(N + off, dtype=torch.float32, device="cuda")
        buf_b = torch.zeros(N + off, dtype=torch.float32, device="cuda")
        buf_a[off:] = dla[bb, tt]
        buf_b[off:] = dlb[bb, tt]
        i1 = torch.empty((1, 1), dtype=torch.int32, device="cuda")
        lp1 = torch.empty((1, 1), dtype=torch.float32, device="cuda")
        xv.xv_greedy_accept(buf_a[off:].view(1, 1, N), buf_b[off:].view(1, 1, N), draft[:1, :1].contiguous(),
                            i1, nk[:1].contiguous(), lp1)
        torch.cuda.synchronize()
        assert int(i1[0, 0]) == int(ids[bb, tt]) and same_bits(lp1[0], lp[bb, tt:tt + 1]), off


# ---------------------------------------------------------------------------
# composed decoding
# ---------------------------------------------------------------------------
def _decoder(name, n_tokens, k_max, S0_from_oracle=True):
    from bit_exact_speculative_amd.decode import Decoder
    wl = gen.WORKLOADS[name]
    inp = gen.composed_inputs(wl)
    S0 = prefix_state(inp) if S0_from_oracle else None
    Lmax = int(inp.L0.max()) + n_tokens + k_max + 2
    return Decoder(inp, Lmax, S0=S0), inp, S0


def _drafts_from(ref, wl, p_wrong, seed):
    rng = np.random.default_rng(seed)
    n = ref.shape[1]

    def drafts(b, pos, k):
        d = np.array([ref[b, min(pos + i, n - 1)] for i in range(k)], np.int32)
        bad = rng.random(k) < p_wrong
        d[bad] = (d[bad] + 1 + rng.integers(0, wl.NH - 1, int(bad.sum()))) % wl.NH
        return d
    return drafts


@pytest.mark.parametrize("name,n,k,p_wrong", [("tiny", 16, 4, 0.3), ("tiny", 12, 8, 1.0),
                                              ("short", 12, 8, 0.3), ("batch8", 10, 8, 0.4)])
def test_speculative_decoding_equals_plain_decoding(name, n, k, p_wrong):
    """The post's claim on the composed step: the same ids and logprobs (and the same
    GDN state and KV cache once the same tokens are consumed) with and without drafts."""
    dec_a, inp, _ = _decoder(name, n + 2 * k, k)
    root = inp.extra["root"]
    ids_a, lp_a, _ = dec_a.generate(root, n + k)          # a reference long enough for the drafts
    dec_b, _, _ = _decoder(name, n + 2 * k, k)
    ids_b, lp_b, keeps = dec_b.generate(root, n, _drafts_from(ids_a, inp.wl, p_wrong, 7), k=k)
    assert np.array_equal(ids_a[:, :n], ids_b)
    assert np.array_equal(lp_a[:, :n].view(np.int32), lp_b.view(np.int32))
    if p_wrong == 1.0:
        assert all(int(x.max()) == 1 for x in keeps)
    else:
        assert max(int(x.max()) for x in keeps) > 1       # some drafts were accepted
    # state after the same consumed tokens: replay plain decoding to the speculative length
    emitted = (dec_b.kv_len - torch.from_numpy(inp.L0).cuda()).cpu().numpy()
    if len(set(emitted.tolist())) == 1:
        dec_c, _, _ = _decoder(name, n + 2 * k, k)
        dec_c.generate(root, int(emitted[0]))
        torch.cuda.synchronize()
        assert same_bits(dec_c.S, dec_b.S) and torch.equal(dec_c.kv_len, dec_b.kv_len)
        L = int(dec_b.kv_len.max())
        assert same_bits(dec_c.Kc[:, :, :L], dec_b.Kc[:, :, :L]) and same_bits(dec_c.Vc[:, :, :L], dec_b.Vc[:, :, :L])


def test_composed_decoding_vs_oracle_tiny():
    """GPU decoding against the oracle's composed decoding from the same start state:
    the ids agree while the oracle's top-2 logit gap stays above what the fp32 path can
    move, and the logprobs agree within the tolerance of the head outputs."""
    n, k = 12, 4
    dec, inp, S0 = _decoder("tiny", n + 2 * k, k)
    wl = inp.wl
    root = inp.extra["root"]
    ids_g, lp_g, _ = dec.generate(root, n)
    s = OC.Shapes(wl.Hk, wl.Hv, wl.dk, wl.dv, wl.Hq, wl.Hkv, wl.d)
    m = OC.Model(inp.extra["E"], inp.W1, inp.W2, inp.Wh_gdn, inp.Wh_attn, s)
    st = OC.State(S0.copy(), inp.k_cache.copy(), inp.v_cache.copy(), inp.L0.copy())
    Lmax = dec.Lmax
    pad = np.zeros((wl.B, wl.Hkv, Lmax - st.kc.shape[2], wl.d), np.uint16)
    st.kc = np.concatenate([st.kc, pad], axis=2)
    st.vc = np.concatenate([st.vc, pad], axis=2)
    ids_o, lp_o, _, gaps = OC.generate(m, st, root, n)
    # the logits' scale: compare in the steps before the first small margin
    good = 0
    for t in range(n):
        if gaps[t].min() < 1e-3:
            break
        good += 1
    assert good >= 4, "margins too small to compare"
    assert np.array_equal(ids_g[:, :good], ids_o[:, :good])
    assert np.all(np.abs(lp_g[:, :good] - lp_o[:, :good]) <= 2e-3 * np.maximum(np.abs(lp_o[:, :good]), 1.0))


def test_divergence_exact_run_never_flips_tiny():
    """Tiny shapes: the exact speculative run equals plain decoding over 256 tokens, 3 seeds."""
    from bit_exact_speculative_amd.diagnose import divergence_margins
    inp = gen.composed_inputs(gen.WORKLOADS["tiny"])
    r = divergence_margins("tiny", n_tokens=256, k=8, p_wrong=0.3, seeds=(0, 1, 2), S0=prefix_state(inp),
                           variants=())
    assert r["exact_spec_diverged"] == 0 and r["requests"] == 3


@pytest.mark.parametrize("name,seeds", [("batch8", (0, 1, 2, 3))])
def test_divergence_margin_diagnostic(name, seeds):
    """The exact speculative run never leaves plain decoding.  Each non-exact variant (fp32
    library product for the verify projections; beta at bf16 in the verify recurrence)
    flips ids over 256 tokens per request, and at every flip the reference's top-1/top-2
    margin is within what the variant's logit perturbation there can bridge (a flip needs
    margin <= 2 x change); the flips sit at the small end of the margins seen."""
    from bit_exact_speculative_amd.diagnose import divergence_margins
    inp = gen.composed_inputs(gen.WORKLOADS[name])
    r = divergence_margins(name, n_tokens=256, k=8, p_wrong=0.3, seeds=seeds, S0=prefix_state(inp))
    assert r["exact_spec_diverged"] == 0
    assert r["requests"] == gen.WORKLOADS[name].B * len(seeds)
    for v, rv in r["variants"].items():
        assert rv["diverged"] > 0, v                    # the diagnostic must see flips to say anything
        assert rv["flips_within_perturbation"], v
        assert max(rv["flip_margin_percentiles"]) < 5.0, v


def test_lazy_rollback_decoding_equals_eager():
    """Decoding with each rollback folded into the next step's GDN launch gives the ids,
    logprobs, state, KV cache and lengths of verify + rollback per step, bit for bit."""
    from bit_exact_speculative_amd.decode import Decoder
    name, n, k = "batch8", 10, 8
    wl = gen.WORKLOADS[name]
    inp = gen.composed_inputs(wl)
    S0 = prefix_state(inp)
    Lmax = int(inp.L0.max()) + n + 2 * k + 2
    ref = Decoder(inp, Lmax, S0=S0, lazy=False)
    root = inp.extra["root"]
    ids_r, _, _ = ref.generate(root, n + k)
    runs = []
    for lazy in (False, True):
        dec = Decoder(inp, Lmax, S0=S0, lazy=lazy)
        ids, lp, keeps = dec.generate(root, n, _drafts_from(ids_r, wl, 0.4, 11), k=k)
        runs.append((ids, lp, keeps, dec.S.clone(), dec.kv_len.clone(), dec.Kc, dec.Vc))
    (i0, l0, k0, S_0, kv0, K0, V0), (i1, l1, k1, S_1, kv1, K1, V1) = runs
    assert np.array_equal(i0, i1) and np.array_equal(l0.view(np.int32), l1.view(np.int32))
    assert all(np.array_equal(a, b) for a, b in zip(k0, k1))
    assert torch.equal(kv0, kv1) and same_bits(S_0, S_1)
    L = int(kv0.max())
    assert same_bits(K0[:, :, :L], K1[:, :, :L]) and same_bits(V0[:, :, :L], V1[:, :, :L])
