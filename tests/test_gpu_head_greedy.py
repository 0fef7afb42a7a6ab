"""xv_head_greedy_accept: the synthetic head and greedy acceptance in one call give the bits of
xv_gemm_small_m_pair followed by xv_greedy_accept (every output), in the fused launch (one row
tile, K = 5120 or 6144) and in the shapes that run the two calls."""
import numpy as np
import pytest
import torch

from tests.gpu_util import same_bits

pytestmark = pytest.mark.gpu


def _inputs(B, T, N, K, seed, ties=False):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    M = B * T
    xa = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    xb = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    if ties:
        # columns n and n + 37 share a weight row in each half: equal logits, lowest index wins
        base_a = (torch.randn((37, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        base_b = (torch.randn((37, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        idx = torch.arange(N, device="cuda") % 37
        wa, wb = base_a[idx].contiguous(), base_b[idx].contiguous()
    else:
        wa = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        wb = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    return xa, wa, xb, wb


def _reference(xa, wa, xb, wb, draft, kv0):
    import bit_exact_speculative_amd.xv as xv
    B, T = draft.shape
    M, N = xa.shape[0], wa.shape[0]
    out = {"ya": torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
           "la": torch.empty((M, N), dtype=torch.float32, device="cuda"),
           "yb": torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
           "lb": torch.empty((M, N), dtype=torch.float32, device="cuda"),
           "ids": torch.empty((B, T), dtype=torch.int32, device="cuda"),
           "nk": torch.empty((B,), dtype=torch.int32, device="cuda"),
           "lp": torch.empty((B, T), dtype=torch.float32, device="cuda"),
           "kv": kv0.clone()}
    xv.xv_gemm_small_m_pair(xa, wa, out["ya"], out["la"], xb, wb, out["yb"], out["lb"])
    xv.xv_greedy_accept(out["la"].view(B, T, N), out["lb"].view(B, T, N), draft, out["ids"], out["nk"],
                        out["lp"], kv_len=out["kv"])
    torch.cuda.synchronize()
    return out


def _fused(xa, wa, xb, wb, draft, kv0, ws):
    import bit_exact_speculative_amd.xv as xv
    B, T = draft.shape
    M, N = xa.shape[0], wa.shape[0]
    # outputs start as NaN / -1 so that an unwritten element shows
    out = {"ya": torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"),
           "la": torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"),
           "yb": torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda"),
           "lb": torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda"),
           "ids": torch.full((B, T), -1, dtype=torch.int32, device="cuda"),
           "nk": torch.full((B,), -1, dtype=torch.int32, device="cuda"),
           "lp": torch.full((B, T), float("nan"), dtype=torch.float32, device="cuda"),
           "kv": kv0.clone()}
    xv.xv_head_greedy_accept(xa, wa, out["ya"], out["la"], xb, wb, out["yb"], out["lb"], draft, out["ids"],
                             out["nk"], ws, logprob=out["lp"], kv_len=out["kv"])
    torch.cuda.synchronize()
    return out


def _drafts(ids_ref, N, seed):
    """Drafts that accept a random prefix of each request's rows (then one mismatch)."""
    rng = np.random.default_rng(seed)
    B, T = ids_ref.shape
    draft = rng.integers(0, N, size=(B, T)).astype(np.int32)
    for b in range(B):
        a = int(rng.integers(0, T))
        for t in range(a):
            draft[b, t + 1] = ids_ref[b, t]
        if a + 1 < T:
            draft[b, a + 1] = (ids_ref[b, a] + 1) % N
    return torch.from_numpy(draft).cuda()


def _check(B, T, N, K, seed, ws=None, ties=False):
    import bit_exact_speculative_amd.xv as xv
    xa, wa, xb, wb = _inputs(B, T, N, K, seed, ties)
    kv0 = torch.arange(100, 100 + B, dtype=torch.int32, device="cuda")
    zero = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    first = _reference(xa, wa, xb, wb, zero, kv0)
    draft = _drafts(first["ids"].cpu().numpy(), N, seed)
    ref = _reference(xa, wa, xb, wb, draft, kv0)
    if ws is None:
        ws = torch.zeros((xv.xv_head_greedy_workspace_bytes(B, T, N),), dtype=torch.uint8, device="cuda")
    got = _fused(xa, wa, xb, wb, draft, kv0, ws)
    for k in ("ya", "la", "yb", "lb", "ids", "nk", "lp", "kv"):
        assert same_bits(got[k], ref[k]), (k, B, T, N, K)
    # the counter is back at zero for the next call
    assert int(ws[:256].to(torch.int32).abs().sum()) == 0
    return ref


# fused launch: B*T <= 16, K = 5120 or 6144; N from one block to more blocks than CUs, and
# block counts that leave chains empty (N / 16 < 256) or give chains two blocks (> 256)
@pytest.mark.parametrize("B,T,N,K", [
    (1, 9, 4096, 6144), (1, 9, 4096, 5120), (1, 16, 4096, 6144), (2, 8, 4096, 6144),
    (16, 1, 4096, 6144), (1, 1, 4096, 6144), (1, 9, 16, 6144), (3, 5, 1008, 5120),
    (1, 9, 4144, 6144), (2, 5, 16384, 5120)])
def test_head_greedy_fused_equals_pair_then_greedy(B, T, N, K):
    _check(B, T, N, K, seed=B * 7919 + T * 131 + N + K)


def test_head_greedy_fused_ties_lowest_index():
    """Logits with many exact ties (repeated weight rows): ids, acceptance and logprobs agree."""
    ref = _check(1, 9, 4096, 6144, seed=11, ties=True)
    ids = ref["ids"].cpu().numpy()
    assert (ids < 37).all()                      # every maximum's lowest copy is in the first 37 columns


@pytest.mark.parametrize("B,T,N,K", [(8, 9, 4096, 6144), (1, 9, 4096, 4096), (1, 10, 64, 64)])
def test_head_greedy_unfused_shapes(B, T, N, K):
    """Shapes outside the fused launch (several row tiles, other K) run the two calls."""
    _check(B, T, N, K, seed=B + T + N + K)


def test_head_greedy_workspace_reused_across_calls():
    """One workspace for consecutive calls of different sizes: each call leaves its counter at
    zero, so the next one (smaller or larger) needs no clearing."""
    import bit_exact_speculative_amd.xv as xv
    ws = torch.zeros((xv.xv_head_greedy_workspace_bytes(2, 8, 4096),), dtype=torch.uint8, device="cuda")
    for (B, T), seed in (((1, 9), 1), ((1, 4), 2), ((2, 8), 3), ((1, 9), 4)):
        _check(B, T, 4096, 6144, seed=seed, ws=ws)


def test_head_greedy_unfused_workspace_reused_across_calls():
    """The unfused path's per-request counters (argmax and acceptance in one launch) are left at
    zero by every call: consecutive calls of different batch sizes on one workspace."""
    import bit_exact_speculative_amd.xv as xv
    ws = torch.zeros((xv.xv_head_greedy_workspace_bytes(8, 9, 4096),), dtype=torch.uint8, device="cuda")
    for (B, T), seed in (((8, 9), 5), ((3, 4), 6), ((8, 9), 7), ((1, 16), 8)):
        _check(B, T, 4096, 4096, seed=seed, ws=ws)

