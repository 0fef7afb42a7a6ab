"""Prefill on the GPU (Decoder.prefill): the prompt through the layer with every row
kept, in chunks.  It must leave the GDN state, KV cache and length of feeding the
prompt one token at a time, bit for bit, and give the same first token and
logprob, for any chunk size and step size; against the oracle's prefill it agrees
within the composed step's tolerances."""
import numpy as np
import pytest
import torch

import oracle
from oracle import compose as C
from bit_exact_speculative_amd import inputs as gen
from tests.gpu_util import STATE_REL_L2, prefix_state, rel_l2, same_bits

pytestmark = pytest.mark.gpu


def _decoder(name, extra, S0=None):
    from bit_exact_speculative_amd.decode import Decoder
    wl = gen.WORKLOADS[name]
    inp = gen.composed_inputs(wl)
    Lmax = int(inp.L0.max()) + extra
    return Decoder(inp, Lmax, S0=S0), inp, wl


def _prompt(wl, P, seed):
    return np.random.default_rng(seed).integers(0, wl.NH, size=(wl.B, P)).astype(np.int32)


def _state(dec):
    L = int(dec.kv_len.max())
    return dec.S.clone(), dec.Kc[:, :, :L].clone(), dec.Vc[:, :, :L].clone(), dec.kv_len.clone()


def _one_token_at_a_time(dec, prompt):
    for t in range(prompt.shape[1]):
        R = dec.step(torch.from_numpy(prompt[:, t:t + 1].copy()).cuda())
    return R.ids[:, 0].clone(), R.lp[:, 0].clone()


@pytest.mark.parametrize("name,P,chunk", [("tiny", 37, 8192), ("tiny", 37, 10), ("short", 45, 16),
                                         ("short", 300, 128), ("batch8", 21, 8)])
def test_prefill_equals_one_token_decoding(name, P, chunk):
    dec_a, inp, wl = _decoder(name, P + 8)
    prompt = _prompt(wl, P, P + chunk)
    id_a, lp_a = dec_a.prefill(prompt, chunk=chunk)
    torch.cuda.synchronize()
    dec_b, _, _ = _decoder(name, P + 8)
    id_b, lp_b = _one_token_at_a_time(dec_b, prompt)
    torch.cuda.synchronize()
    assert torch.equal(id_a, id_b) and same_bits(lp_a, lp_b)
    Sa, Ka, Va, la = _state(dec_a)
    Sb, Kb, Vb, lb = _state(dec_b)
    assert torch.equal(la, lb) and torch.equal(la.cpu(), torch.from_numpy(inp.L0 + P))
    assert same_bits(Sa, Sb) and same_bits(Ka, Kb) and same_bits(Va, Vb)


def test_prefill_then_speculative_decoding_equals_plain_decoding():
    """After a prefill, decoding with drafts and without them emits the same ids and logprobs."""
    dec_a, inp, wl = _decoder("tiny", 30 + 40)
    prompt = _prompt(wl, 30, 3)
    first, _ = dec_a.prefill(prompt)
    root = first.cpu().numpy()
    snap = dec_a.snapshot()
    ids_p, lp_p, _ = dec_a.generate(root, 20)
    dec_a.restore(snap)
    rng = np.random.default_rng(5)

    def drafts(b, pos, k):
        d = np.array([ids_p[b, min(pos + i, 19)] for i in range(k)], np.int32)
        bad = rng.random(k) < 0.3
        d[bad] = (d[bad] + 1) % wl.NH
        return d
    ids_s, lp_s, _ = dec_a.generate(root, 12, drafts, k=6)
    assert np.array_equal(ids_s, ids_p[:, :12]) and np.array_equal(lp_s.view(np.int32), lp_p[:, :12].view(np.int32))


def test_prefill_vs_oracle_tiny():
    """The GPU prefill against the oracle's from the same start state (the oracle's own
    prefix state): the state within the GDN tolerance, the first token where the oracle's
    top-2 gap leaves no doubt, its logprob within 2e-3 relative, the cache rows within one
    bf16 rounding of the oracle's."""
    wl = gen.WORKLOADS["tiny"]
    inp = gen.composed_inputs(wl)
    S0 = prefix_state(inp)
    P = 40
    dec, _, _ = _decoder("tiny", P + 8, S0=S0)
    prompt = _prompt(wl, P, 11)
    id_g, lp_g = dec.prefill(prompt, chunk=16)
    torch.cuda.synchronize()
    s = C.Shapes(wl.Hk, wl.Hv, wl.dk, wl.dv, wl.Hq, wl.Hkv, wl.d)
    m = C.Model(inp.extra["E"], inp.W1, inp.W2, inp.Wh_gdn, inp.Wh_attn, s)
    Lmax = dec.Kc.shape[2]
    kc = np.zeros((wl.B, wl.Hkv, Lmax, wl.d), np.uint16)
    vc = np.zeros_like(kc)
    L0 = int(inp.L0[0])
    kc[:, :, :L0] = inp.k_cache[:, :, :L0]
    vc[:, :, :L0] = inp.v_cache[:, :, :L0]
    st = C.State(S0.astype(np.float32).copy(), kc, vc, inp.L0.copy())
    id_o, lp_o, z_o = C.prefill(m, st, prompt)
    srt = np.sort(z_o, axis=-1)
    for bb in range(wl.B):
        if srt[bb, -1] - srt[bb, -2] > 1e-3:
            assert int(id_g[bb]) == int(id_o[bb])
            assert abs(float(lp_g[bb]) - lp_o[bb]) <= 2e-3 * max(abs(lp_o[bb]), 1e-3) + 1e-5
    # q, k, v reach the state after a bf16 rounding of an fp32 (GPU) or fp64 (oracle) value; a
    # rounding that falls on the other side of a tie moves one element by one bf16 ulp, so the
    # state is held to ten times the GDN-only bound
    assert rel_l2(dec.S.cpu().numpy(), st.S) <= STATE_REL_L2 * 10
    L = L0 + P
    kg = dec.Kc[:, :, L0:L].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ko = st.kc[:, :, L0:L]
    diff = np.abs(C.bf16_value(kg) - C.bf16_value(ko))
    assert np.all(diff <= 2.0 ** -7 * np.abs(C.bf16_value(ko)) + 1e-30)
