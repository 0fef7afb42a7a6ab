"""Run-to-run repeatability at the post's scale and capacity invariance at the launch
command's context length.

The post's repeatability paragraph: without the DeepGEMM fence, 25 of 1,200 requests sent in
batches of 8 came out different; with it, none.  Here the kernels that hand partial results
from workgroup to workgroup (the greedy acceptance's per-request counters, the batch-1 head's
greedy tail, the per-tile attention fold) do so through device-coherent stores, loads and
counters in each caller's own workspace, with fixed fold orders, so 1,200 full lazy steps of a
batch of 8 (and of batch 1) must give every bit twice, also when two copies of the layer run at
the same time on two streams.  The launch command sets a
262,144-token context: a cache of that capacity must give the bits of a cache of exactly
the verified length."""
import numpy as np
import pytest
import torch

from bit_exact_speculative_amd import inputs as gen
from tests.gpu_util import prefix_state, same_bits

pytestmark = pytest.mark.gpu

STEPS = 1200
RESET_EVERY = 100          # steps between returns to the pre-verify caches (bounds the capacity)


@pytest.mark.parametrize("workload", ["batch8", "short"])
def test_repeatability_1200_steps_two_streams(workload):
    """Two copies of the layer (batch 8, or batch 1 with the fused head tail and the per-tile
    attention fold), 1,200 full lazy steps each (projections, GDN after the previous step's
    rollback beside attention with the KV append, head, greedy acceptance), step k of copy A on
    stream k % 2 and of copy B on the other stream, both in flight together: ids, logprobs,
    projection, GDN and attention outputs equal at every step, states and caches equal at
    every reset.  Stops at the first difference."""
    from bit_exact_speculative_amd.layer import Layer
    wl = gen.WORKLOADS[workload]
    L0max = wl.L0 if wl.L0 is not None else wl.L0_range[1]
    Lmax = L0max + wl.T * (RESET_EVERY + 4)
    inp = gen.make_inputs(wl, Lmax=Lmax, pad_value=0)
    S0 = prefix_state(inp)
    A = Layer(inp, "cuda", state_in=S0)
    A.proj_fp32 = False
    A.out_fp32 = False
    B = A.clone()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    done = {"A": None, "B": None}           # each copy's last step event (its next step waits on it)

    def run(L, key, s):
        if done[key] is not None:
            s.wait_event(done[key])
        with torch.cuda.stream(s):
            L.lazy_step()
        ev = torch.cuda.Event()
        ev.record(s)
        done[key] = ev

    for k in range(STEPS):
        run(A, "A", streams[k % 2])
        run(B, "B", streams[(k + 1) % 2])
        torch.cuda.synchronize()
        assert torch.equal(A.ids, B.ids) and same_bits(A.lp, B.lp), k
        assert same_bits(A.y1, B.y1) and same_bits(A.y2, B.y2), k
        assert same_bits(A.o_gdn, B.o_gdn) and same_bits(A.o_attn, B.o_attn), k
        assert torch.equal(A.kv_len, B.kv_len) and torch.equal(A.n_keep, B.n_keep), k
        if (k + 1) % RESET_EVERY == 0:
            for L in (A, B):
                L.settle()
                torch.cuda.synchronize()
            assert same_bits(A.S_in, B.S_in) and same_bits(A.Kc, B.Kc) and same_bits(A.Vc, B.Vc), k
            for L in (A, B):
                L.reset()
            torch.cuda.synchronize()
            done = {"A": None, "B": None}


def test_capacity_262144_gives_the_bits_of_the_exact_capacity():
    """The short workload (640 cached tokens, 9 rows) verified in a 262,144-position cache
    (slots past the rows hold a NaN, never read) and in a cache of exactly 649 positions:
    GDN, attention, head logits and ids, and the appended cache rows are bit-identical.  The
    large capacity takes the streaming partial kernel and the long-row combine; the exact one
    the per-tile kernel and the short-row combine."""
    from bit_exact_speculative_amd.layer import Layer
    wl = gen.WORKLOADS["short"]
    small = gen.make_inputs(wl)                       # the head weights follow the projections' draws
    big = gen.make_inputs(wl, Lmax=262144)
    S0 = prefix_state(small)
    out = []
    for inp in (small, big):
        L = Layer(inp, "cuda", state_in=S0, with_gemm=False)
        L.verify(rollback=False)
        torch.cuda.synchronize()
        m = int(inp.L0[0]) + wl.T
        out.append((L.o_gdn32.clone(), L.o_attn.clone(), L.o_attn32.clone(), L.lg32.clone(), L.la32.clone(),
                    L.ids.clone(), L.S_out.clone(), L.Kc[:, :, :m].clone(), L.Vc[:, :, :m].clone()))
        del L
        torch.cuda.empty_cache()
    for i, (a, b) in enumerate(zip(*out)):
        assert same_bits(a, b), i
