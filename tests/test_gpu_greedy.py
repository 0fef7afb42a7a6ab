"""xv_greedy_accept on the GPU against the oracle's greedy rule on identical logits."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


def _run(la, lb, draft):
    import bit_exact_speculative_amd.xv as xv
    B, T, N = la.shape
    dla = torch.from_numpy(la).cuda()
    dlb = torch.from_numpy(lb).cuda() if lb is not None else None
    dd = torch.from_numpy(draft).cuda()
    ids = torch.empty((B, T), dtype=torch.int32, device="cuda")
    nk = torch.empty((B,), dtype=torch.int32, device="cuda")
    xv.xv_greedy_accept(dla, dlb, dd, ids, nk)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), nk.cpu().numpy()


@pytest.mark.parametrize("B,T,N", [(1, 9, 4096), (8, 9, 4096), (2, 1, 4096), (3, 16, 1000),
                                   (1, 5, 7), (2, 4, 4100), (1, 16, 1), (1, 12, 12288)])
@pytest.mark.parametrize("two", [False, True])
def test_greedy_matches_oracle(B, T, N, two):
    rng = np.random.default_rng(B * 1000 + T * 10 + N)
    # few distinct values so that ties are common
    la = rng.integers(-3, 4, size=(B, T, N)).astype(np.float32) * np.float32(0.5)
    lb = rng.integers(-2, 3, size=(B, T, N)).astype(np.float32) * np.float32(0.25) if two else None
    logits = la + lb if two else la                      # the same fp32 sum the kernel forms
    ids_ref, _ = oracle.greedy(logits.astype(np.float64), np.zeros((B, T), np.int32))
    # drafts that accept a known prefix per request
    draft = rng.integers(0, N, size=(B, T)).astype(np.int32)
    want = []
    for bb in range(B):
        a = int(rng.integers(0, T))
        for t in range(a):
            draft[bb, t + 1] = ids_ref[bb, t]
        if a + 1 < T:
            draft[bb, a + 1] = (ids_ref[bb, a] + 1) % max(N, 2) if N > 1 else ids_ref[bb, a]
        want.append(a)
    ids_ref, nk_ref = oracle.greedy(logits.astype(np.float64), draft)
    ids, nk = _run(la, lb, draft)
    assert np.array_equal(ids, ids_ref)
    assert np.array_equal(nk, nk_ref)


def test_greedy_scalar_path_on_unaligned_rows():
    """A logits view that starts 4 bytes into its buffer takes the 4-byte-load path."""
    import bit_exact_speculative_amd.xv as xv
    rng = np.random.default_rng(5)
    B, T, N = 1, 9, 4096
    big = rng.standard_normal(B * T * N + 1).astype(np.float32)
    dev = torch.from_numpy(big).cuda()
    la = dev[1:].view(B, T, N)
    draft = torch.zeros((B, T), dtype=torch.int32, device="cuda")
    ids = torch.empty((B, T), dtype=torch.int32, device="cuda")
    nk = torch.empty((B,), dtype=torch.int32, device="cuda")
    xv.xv_greedy_accept(la, None, draft, ids, nk)
    torch.cuda.synchronize()
    ref, _ = oracle.greedy(big[1:].reshape(B, T, N).astype(np.float64), np.zeros((B, T), np.int32))
    assert np.array_equal(ids.cpu().numpy(), ref)
