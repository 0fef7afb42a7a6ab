"""The whole verify step of one hybrid layer on the GPU, on the five workloads:
verify == k+1 sequential decode steps in every output bit and in the greedy ids;
forced reject restores the pre-verify state and length bit for bit; a batch of 8
gives each request its batch-1 bits; long context; oracle parity throughout."""
import numpy as np
import pytest
import torch

import oracle
from bit_exact_speculative_amd.inputs import f32_to_bf16_bits
from tests.gpu_util import OUT_MAX_REL, STATE_REL_L2, max_rel, rel_l2, same_bits, workload

pytestmark = pytest.mark.gpu


def _layer(name, gemm=True, head=True):
    from bit_exact_speculative_amd.layer import Layer
    inp, S0 = workload(name, gemm, head)
    return Layer(inp, "cuda", state_in=S0), inp, S0


def _check_verify_equals_decode(L, dec, n_rows=None):
    B, T = L.B, L.T
    n = T if n_rows is None else n_rows
    assert same_bits(L.o_gdn[:, :n], dec["o_gdn"]) and same_bits(L.o_gdn32[:, :n], dec["o_gdn32"])
    assert same_bits(L.o_attn[:, :n], dec["o_attn"]) and same_bits(L.o_attn32[:, :n], dec["o_attn32"])
    if L.has_gemm:
        wl = L.wl
        assert same_bits(L.y1_32.view(B, T, wl.N1)[:, :n], dec["y1_32"])
        assert same_bits(L.y2_32.view(B, T, wl.N2)[:, :n], dec["y2_32"])
        assert same_bits(L.y1.view(B, T, wl.N1)[:, :n], dec["y1"])
    if L.has_head:
        assert same_bits(L.lg32.view(B, T, -1)[:, :n], dec["lg32"])
        assert same_bits(L.la32.view(B, T, -1)[:, :n], dec["la32"])
        assert torch.equal(L.ids[:, :n], dec["ids"])
        assert same_bits(L.lp[:, :n], dec["lp"])


def _oracle_ids_consistent(L, inp, S0):
    """GPU ids may differ from the fp64 oracle's only where the oracle's own top-1 margin
    is within the error the tolerances allow."""
    wl = inp.wl
    g = inp.gdn
    o_ref, _, _ = oracle.gdn(g["q"], g["k"], g["v"], g["a"], g["b"], S0)
    a_ref = oracle.attn(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0, L.scale)
    fg = f32_to_bf16_bits(o_ref.astype(np.float32)).reshape(wl.M, -1)
    fa = f32_to_bf16_bits(a_ref.astype(np.float32)).reshape(wl.M, -1)
    logits = oracle.gemm(fg, inp.Wh_gdn) + oracle.gemm(fa, inp.Wh_attn)
    ids_ref, _ = oracle.greedy(logits.reshape(wl.B, wl.T, wl.NH), inp.draft)
    ids = L.ids.cpu().numpy()
    wg = np.abs((inp.Wh_gdn.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    wa = np.abs((inp.Wh_attn.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    # |delta feature| <= (2^-8 + 2e-3) |f| per element (bf16 rounding + output tolerance)
    rel = 2.0 ** -8 + OUT_MAX_REL
    bound = wg @ (np.abs(o_ref.reshape(wl.M, -1)) * rel).T + wa @ (np.abs(a_ref.reshape(wl.M, -1)) * rel).T
    bound = bound.T.reshape(wl.B, wl.T, wl.NH)
    lg = logits.reshape(wl.B, wl.T, wl.NH)
    for bb in range(wl.B):
        for t in range(wl.T):
            i_g, i_r = ids[bb, t], ids_ref[bb, t]
            if i_g != i_r:
                gap = lg[bb, t, i_r] - lg[bb, t, i_g]
                assert gap <= bound[bb, t, i_r] + bound[bb, t, i_g], (bb, t, gap)


@pytest.mark.parametrize("name", ["tiny", "short"])
def test_step_verify_equals_decode(name):
    L, inp, S0 = _layer(name)
    L.verify(rollback=False)
    dec = L.decode_sequence()
    torch.cuda.synchronize()
    _check_verify_equals_decode(L, dec)
    assert same_bits(L.S_out, dec["S"][-1])
    assert same_bits(L.Kc, dec["Kc"]) and same_bits(L.Vc, dec["Vc"])
    # oracle parity of the three parts
    g = inp.gdn
    o_ref, S_ref, _ = oracle.gdn(g["q"], g["k"], g["v"], g["a"], g["b"], S0)
    assert rel_l2(L.S_out.cpu().numpy(), S_ref) <= STATE_REL_L2
    assert max_rel(L.o_gdn32.cpu().numpy(), o_ref) <= OUT_MAX_REL
    a_ref = oracle.attn(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0, L.scale)
    assert max_rel(L.o_attn32.cpu().numpy(), a_ref) <= OUT_MAX_REL
    if name == "tiny":
        assert max_rel(L.y1_32.cpu().numpy(), oracle.gemm(inp.x, inp.W1)) <= OUT_MAX_REL
    _oracle_ids_consistent(L, inp, S0)


def test_step_forced_reject_restores_pre_verify_bits():
    """Medium context: reject every draft (0 rows kept) -> S and kv_len are the pre-verify bits;
    keep 1 row -> exactly one decode step; keep any n -> n decode steps."""
    L, inp, S0 = _layer("medium", gemm=False, head=False)
    dec = L.decode_sequence()
    S_pre = L.S_in.clone()
    for n in [0, 1, 5, L.T]:
        L.reset()
        L.verify(rollback=False)
        L.rollback(torch.full((1,), n, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert L.kv_len.tolist() == [int(inp.L0[0]) + n]
        want = S_pre if n == 0 else dec["S"][n - 1]
        assert same_bits(L.S_out, want), n
        # the cache below the new length equals the one sequential decode built
        m = int(inp.L0[0]) + n
        assert same_bits(L.Kc[:, :, :m], dec["Kc"][:, :, :m]) and same_bits(L.Vc[:, :, :m], dec["Vc"][:, :, :m])
    Sn, _ = oracle.rollback(inp.gdn["k"], inp.gdn["v"], inp.gdn["a"], inp.gdn["b"], S0, inp.L0,
                            np.array([L.T], np.int32))
    assert rel_l2(L.S_out.cpu().numpy(), Sn) <= STATE_REL_L2


def test_step_batch8_equals_batch1():
    """8 requests in flight (contexts 560..740, accepted lengths 0..8): each request's outputs,
    rolled-back state and length equal its own batch-1 run; GEMM M = 72 rows equal M = 9."""
    from bit_exact_speculative_amd.layer import Layer
    L, inp, S0 = _layer("batch8", gemm=True, head=False)
    n_keep = torch.from_numpy(inp.accepted + 1).cuda()
    L.verify(n_keep=n_keep)
    torch.cuda.synchronize()
    wl = inp.wl
    for bb in range(wl.B):
        sub = _slice_inputs(inp, bb)
        L1 = Layer(sub, "cuda", state_in=S0[bb:bb + 1])
        L1.verify(n_keep=n_keep[bb:bb + 1].clone())
        torch.cuda.synchronize()
        assert same_bits(L1.o_gdn32[0], L.o_gdn32[bb]) and same_bits(L1.o_attn32[0], L.o_attn32[bb])
        assert same_bits(L1.S_out[0], L.S_out[bb]) and L1.kv_len.item() == L.kv_len[bb].item()
        assert same_bits(L1.y1_32, L.y1_32[bb * 9:(bb + 1) * 9])
        assert same_bits(L1.y2, L.y2[bb * 9:(bb + 1) * 9])
        Lk = int(inp.L0[bb]) + int(n_keep[bb])
        assert same_bits(L1.Kc[0, :, :Lk], L.Kc[bb, :, :Lk])
        del L1
    g = inp.gdn
    Sn, kv = oracle.rollback(g["k"], g["v"], g["a"], g["b"], S0, inp.L0, inp.accepted + 1)
    assert rel_l2(L.S_out.cpu().numpy(), Sn) <= STATE_REL_L2
    assert L.kv_len.cpu().numpy().tolist() == kv.tolist()


def _slice_inputs(inp, bb):
    import copy
    from bit_exact_speculative_amd.inputs import Inputs, Workload
    wl = inp.wl
    w1 = Workload(**{**wl.__dict__, "B": 1, "name": wl.name + "_r%d" % bb})
    sl = slice(bb, bb + 1)
    return Inputs(wl=w1, prefix={k: v[sl] for k, v in inp.prefix.items()},
                  gdn={k: v[sl] for k, v in inp.gdn.items()}, L0=inp.L0[sl].copy(), Lmax=inp.Lmax,
                  q_attn=inp.q_attn[sl], k_new=inp.k_new[sl], v_new=inp.v_new[sl],
                  k_cache=inp.k_cache[sl], v_cache=inp.v_cache[sl],
                  x=inp.x[bb * wl.T:(bb + 1) * wl.T], W1=inp.W1, W2=inp.W2)


def test_step_long_context():
    """127735 cached tokens: attention verify rows == decode rows; sampled rows vs the oracle;
    GEMM and GDN rows at M = 1 equal their M = 9 bits."""
    L, inp, S0 = _layer("long", gemm=True, head=False)
    L.verify(rollback=False)
    dec = L.decode_sequence()
    torch.cuda.synchronize()
    _check_verify_equals_decode(L, dec)
    assert same_bits(L.S_out, dec["S"][-1])
    o32 = L.o_attn32.cpu().numpy()
    for (r, h) in [(0, 0), (4, 7), (8, 23), (8, 5), (2, 18)]:
        ref = oracle.attn_row(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0,
                              L.scale, 0, r, h)
        assert max_rel(o32[0, r, h], ref) <= OUT_MAX_REL, (r, h)
