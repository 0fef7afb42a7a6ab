"""The speculative step exactly as the throughput benchmark launches it, at full sizes
(5120-wide projections, 48 GDN heads, 24 query heads, a 4096-wide head) for batch 1 over
640 and 2183 cached tokens, batch 8 over 560-740 and batch 1 over 127,735: the
projection pair in one launch, GDN and attention in one launch where they fit (from the
second step on with the previous step's rollback folded in), the head pair, the greedy
acceptance that also counts the kept KV rows, and the settle after the last step;
bf16-only projection, GDN and attention outputs as in the benchmark.  Every step is
checked against the oracle run on the same inputs from the same state, carried from step
to step with the GPU's acceptance counts (whose rule is checked on the GPU's ids); at
127,735 tokens the attention rows are checked on a sample (the oracle takes one row at a
time there)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.compose import bf16_value
from bit_exact_speculative_amd import inputs as gen
from tests.gpu_util import OUT_MAX_REL, STATE_REL_L2, max_rel, prefix_state, rel_l2, same_bits

pytestmark = pytest.mark.gpu
STEPS = 3
# an output within OUT_MAX_REL of the oracle's, then rounded to bf16 (unit roundoff 2^-8)
BF16_REL = 2.0 ** -8 + OUT_MAX_REL * (1 + 2.0 ** -8)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _sum_bound(x, w):
    """A bound on the error of any fp32 summation order of sum_k x[m][k] w[n][k]:
    gamma_K sum_k |x w| with gamma_K = K u / (1 - K u), u = 2^-24 (the products of two bf16
    values are exact in fp32)."""
    K = x.shape[1]
    u = 2.0 ** -24
    return (K * u / (1 - K * u)) * oracle.gemm(x & 0x7FFF, w & 0x7FFF)


@pytest.mark.parametrize("name", ["short", "medium", "batch8", "long"])
def test_benchmark_step_sequence_vs_oracle(name):
    from bit_exact_speculative_amd.layer import Layer
    wl = gen.WORKLOADS[name]
    B, T, M = wl.B, wl.T, wl.M
    L0max = wl.L0 if wl.L0 is not None else wl.L0_range[1]
    inp = gen.make_inputs(wl, Lmax=L0max + T * (STEPS + 4))
    S0 = prefix_state(inp)
    L = Layer(inp, "cuda", state_in=S0)
    L.proj_fp32 = False
    L.out_fp32 = False
    g = inp.gdn
    S = S0                                        # the oracle's state, handed on in fp32
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    kv = inp.L0.copy()
    y_ref = None
    for s in range(STEPS):
        L.lazy_step()
        torch.cuda.synchronize()
        # projections: the same x every step, so the same bits every step
        y1, y2 = _bits(L.y1), _bits(L.y2)
        if y_ref is None:
            y_ref = (y1, y2)
            assert max_rel(bf16_value(y1), oracle.gemm(inp.x, inp.W1)) <= BF16_REL
            assert max_rel(bf16_value(y2), oracle.gemm(inp.x, inp.W2)) <= BF16_REL
        else:
            assert np.array_equal(y1, y_ref[0]) and np.array_equal(y2, y_ref[1]), s
        # GDN and attention from the oracle's state and cache
        o_ref, _, _ = oracle.gdn(g["q"], g["k"], g["v"], g["a"], g["b"], S)
        fg = _bits(L.o_gdn).reshape(M, -1)
        assert max_rel(bf16_value(fg), o_ref.reshape(M, -1)) <= BF16_REL, s
        fa = _bits(L.o_attn).reshape(M, -1)
        if name == "long":
            fa4 = bf16_value(fa).reshape(B, T, wl.Hq, wl.d)
            for (bb, r, h) in [(0, 0, 0), (0, 8, 23), (0, 4, 11)]:
                ref = oracle.attn_row(inp.q_attn, inp.k_new, inp.v_new, kc, vc, kv, L.scale, bb, r, h)
                assert max_rel(fa4[bb, r, h], ref) <= BF16_REL, (s, bb, r, h)
        else:
            a_ref = oracle.attn(inp.q_attn, inp.k_new, inp.v_new, kc, vc, kv, L.scale)
            assert max_rel(bf16_value(fa), a_ref.reshape(M, -1)) <= BF16_REL, s
        # the head on the GPU's own bf16 features
        lg_ref = oracle.gemm(fg, inp.Wh_gdn)
        la_ref = oracle.gemm(fa, inp.Wh_attn)
        assert max_rel(L.lg32.cpu().numpy(), lg_ref) <= OUT_MAX_REL, s
        assert max_rel(L.la32.cpu().numpy(), la_ref) <= OUT_MAX_REL, s
        logits = (lg_ref + la_ref).reshape(B, T, wl.NH)
        bound = (_sum_bound(fg, inp.Wh_gdn) + _sum_bound(fa, inp.Wh_attn)).reshape(B, T, wl.NH)
        bound += 2.0 ** -24 * np.abs(logits)          # the fp32 sum of the two halves
        ids = L.ids.cpu().numpy()
        ids_ref, _ = oracle.greedy(logits, inp.draft)
        for bb in range(B):
            for t in range(T):
                i_g, i_r = ids[bb, t], ids_ref[bb, t]
                if i_g != i_r:
                    gap = logits[bb, t, i_r] - logits[bb, t, i_g]
                    assert gap <= bound[bb, t, i_r] + bound[bb, t, i_g], (s, bb, t, gap)
        lp_ref = oracle.logprob(logits, ids)
        lp = L.lp.cpu().numpy()
        assert np.all(np.abs(lp - lp_ref) <= 2e-3 * np.maximum(np.abs(lp_ref), 1.0)), s
        # the acceptance rule on the GPU's ids: the oracle's greedy on one-hot logits
        onehot = np.zeros((B, T, wl.NH), np.float64)
        np.put_along_axis(onehot, ids[..., None].astype(np.int64), 1.0, axis=-1)
        _, n_rule = oracle.greedy(onehot, inp.draft)
        n_keep = L.n_keep.cpu().numpy()
        assert np.array_equal(n_keep, n_rule), s
        # the oracle's step ends with the GPU's acceptance: state, cache rows and length
        Sn, kv_next = oracle.rollback(g["k"], g["v"], g["a"], g["b"], S, kv, n_keep)
        for bb in range(B):
            n = int(n_keep[bb])
            kc[bb, :, kv[bb]:kv[bb] + n] = inp.k_new[bb, :n].transpose(1, 0, 2)
            vc[bb, :, kv[bb]:kv[bb] + n] = inp.v_new[bb, :n].transpose(1, 0, 2)
        S, kv = Sn.astype(np.float32), kv_next
        assert np.array_equal(L.kv_len.cpu().numpy(), kv), s
    L.settle()
    torch.cuda.synchronize()
    assert rel_l2(L.S_in.cpu().numpy(), S) <= STATE_REL_L2
    Kg, Vg = _bits(L.Kc), _bits(L.Vc)
    for bb in range(B):                             # each request's cache up to its own length
        n = int(kv[bb])
        assert np.array_equal(Kg[bb, :, :n], kc[bb, :, :n]) and np.array_equal(Vg[bb, :, :n], vc[bb, :, :n]), bb
    assert not same_bits(L.S_in, torch.from_numpy(S0).cuda())     # the state moved
