"""xv_gemm_small_m on the GPU: oracle parity and M / row-position invariance of the bits."""
import numpy as np
import pytest
import torch

import oracle
from bit_exact_speculative_amd.inputs import f32_to_bf16_bits, random_bf16
from tests.gpu_util import OUT_MAX_REL, max_rel, workload

pytestmark = pytest.mark.gpu


def _xv():
    import bit_exact_speculative_amd.xv as xv
    return xv


def _gemm(x_bits, w_bits):
    from bit_exact_speculative_amd.layer import dev_bf16, host_bits
    M, K = x_bits.shape
    N = w_bits.shape[0]
    x = dev_bf16(x_bits, "cuda"); w = dev_bf16(w_bits, "cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    _xv().xv_gemm_small_m(x, w, y, y32)
    torch.cuda.synchronize()
    return host_bits(y), y32.cpu().numpy()


def _gemm_dev(x, w, with32=True):
    M, N = x.shape[0], w.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda") if with32 else None
    _xv().xv_gemm_small_m(x, w, y, y32)
    return y, y32


@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (5, 512, 256), (9, 48, 96), (16, 64, 544),
                                   (17, 32, 1024), (33, 16, 64), (72, 80, 320), (130, 32, 64),
                                   (9, 112, 5120), (9, 48, 6144), (1, 32, 6144)])
def test_gemm_matches_oracle(M, N, K):
    rng = np.random.default_rng(100 + M + N + K)
    x = random_bf16(rng, (M, K))
    w = random_bf16(rng, (N, K), 0.02)
    yb, y32 = _gemm(x, w)
    ref = oracle.gemm(x, w)
    assert max_rel(y32, ref) <= OUT_MAX_REL
    # forward error bound of an fp32 dot product of length K (any summation order)
    xa = np.abs((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    wa = np.abs((w.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    assert np.all(np.abs(y32 - ref) <= 2 * gamma * (xa @ wa.T) + 1e-30)
    assert np.array_equal(yb, f32_to_bf16_bits(y32))          # y is y32 rounded to nearest even


def test_gemm_exact_on_integers():
    """Integer x and w/64: every partial sum is exact in fp32, so y32 must equal the oracle."""
    rng = np.random.default_rng(7)
    M, N, K = 9, 64, 544
    xi = rng.integers(-4, 5, size=(M, K)); wi = rng.integers(-4, 5, size=(N, K))
    x = f32_to_bf16_bits(xi.astype(np.float32))
    w = f32_to_bf16_bits((wi / 64.0).astype(np.float32))
    _, y32 = _gemm(x, w)
    assert np.array_equal(y32.astype(np.float64), oracle.gemm(x, w))


@pytest.mark.parametrize("K", [5120, 6144, 1024])
def test_gemm_row_bits_independent_of_m_and_position(K):
    """Row bits must not depend on M, on the other rows, or on the row's slot in a 16-row tile.

    K = 5120 and 6144 take the LDS-staged kernel for M <= 16 and the row-tile one for M = 72 (at
    K = 5120 its parts of 4 k-steps end a range inside every other part), K = 1024 the
    register-streamed one for M <= 32: the bits must agree across all of them."""
    rng = np.random.default_rng(8 + K)
    N = 96
    from bit_exact_speculative_amd.layer import dev_bf16
    x72 = dev_bf16(random_bf16(rng, (72, K)), "cuda")
    w = dev_bf16(random_bf16(rng, (N, K), 0.02), "cuda")
    ref, ref32 = _gemm_dev(x72, w)
    for M in range(1, 17):
        y, y32 = _gemm_dev(x72[:M].contiguous(), w)
        assert torch.equal(y32.view(torch.int32), ref32[:M].view(torch.int32)), M
        assert torch.equal(y.view(torch.int16), ref[:M].view(torch.int16)), M
    for b in range(8):                                      # one request's 9 rows alone
        y, y32 = _gemm_dev(x72[b * 9:(b + 1) * 9].contiguous(), w)
        assert torch.equal(y32.view(torch.int32), ref32[b * 9:(b + 1) * 9].view(torch.int32)), b
    for m in (0, 5, 15, 16, 40, 71):                         # single rows (decode, M = 1)
        y, y32 = _gemm_dev(x72[m:m + 1].contiguous(), w)
        assert torch.equal(y32.view(torch.int32), ref32[m:m + 1].view(torch.int32)), m
    for shift in (1, 7, 13):                                 # the same rows at other tile slots
        pad = dev_bf16(random_bf16(rng, (shift, K)), "cuda")
        xs = torch.cat([pad, x72[:20]], 0).contiguous()
        y, y32 = _gemm_dev(xs, w)
        assert torch.equal(y32[shift:].view(torch.int32), ref32[:20].view(torch.int32)), shift
    _, none32 = _gemm_dev(x72[:9].contiguous(), w, with32=False)   # y32 = NULL: y unchanged
    y9, _ = _gemm_dev(x72[:9].contiguous(), w)
    assert torch.equal(y9.view(torch.int16), ref[:9].view(torch.int16))


@pytest.mark.parametrize("which", ["N1", "N2"])
def test_gemm_real_shapes_vs_oracle(which):
    """The 27B-class projections (M = 9, K = 5120, N = 10240 / 17408) against the oracle."""
    inp, _ = workload("short", gemm=True, head=False)
    W = inp.W1 if which == "N1" else inp.W2
    yb, y32 = _gemm(inp.x, W)
    ref = oracle.gemm(inp.x, W)
    assert max_rel(y32, ref) <= OUT_MAX_REL
    assert np.array_equal(yb, f32_to_bf16_bits(y32))


def test_gemm_empty_and_repeat():
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(9)
    x = dev_bf16(random_bf16(rng, (9, 256)), "cuda")
    w = dev_bf16(random_bf16(rng, (64, 256), 0.02), "cuda")
    y = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    _xv().xv_gemm_small_m(x[:0], w, y)                       # M = 0: no launch, ok
    first, first32 = _gemm_dev(x, w)
    for _ in range(50):
        y, y32 = _gemm_dev(x, w)
        assert torch.equal(y32.view(torch.int32), first32.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(72, 17408, 5120), (72, 10240, 5120), (33, 16384, 1024), (20, 8192, 544)])
def test_gemm_many_tiles_k_loop_rows_equal_k_split(M, N, K):
    """Wide N with several row tiles runs the K-loop kernel (whole output tiles per wave, ranges
    folded in order); every row must equal the same row computed at M <= 16 by the K-split
    kernels, and sampled columns must match the oracle."""
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(M * 7 + N + K)
    xh = random_bf16(rng, (M, K))
    wh = random_bf16(rng, (N, K), 0.02)
    x = dev_bf16(xh, "cuda"); w = dev_bf16(wh, "cuda")
    y, y32 = _gemm_dev(x, w)
    for r0 in range(0, M, 9):                              # 9-row slices, as one request's rows
        r1 = min(M, r0 + 9)
        ys, ys32 = _gemm_dev(x[r0:r1].contiguous(), w)
        assert torch.equal(ys32.view(torch.int32), y32[r0:r1].view(torch.int32)), r0
        assert torch.equal(ys.view(torch.int16), y[r0:r1].view(torch.int16)), r0
    cols = np.sort(rng.choice(N, size=64, replace=False))
    ref = oracle.gemm(xh, wh[cols])
    torch.cuda.synchronize()
    assert max_rel(y32.cpu().numpy()[:, cols], ref) <= OUT_MAX_REL


def test_gemm_timed_entry_point_same_bits_and_kernel_interval():
    """xv_gemm_small_m_timed: the same bits as xv_gemm_small_m, and its launch-recorded interval is
    positive and no longer than events recorded on the stream around the call."""
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(11)
    xv = _xv()
    x = dev_bf16(random_bf16(rng, (9, 5120)), "cuda")
    w = dev_bf16(random_bf16(rng, (4096, 5120), 0.02), "cuda")
    ref, ref32 = _gemm_dev(x, w)
    for M in (9, 72, 0):
        xm = x[:min(M, 9)].contiguous() if M <= 9 else torch.cat([x] * 8, 0).contiguous()
        y = torch.empty((M, 4096), dtype=torch.bfloat16, device="cuda")
        y32 = torch.empty((M, 4096), dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s = torch.cuda.current_stream()
        e0.record(s); e1.record(s)                   # created
        b0.record(s)
        xv.xv_gemm_small_m_timed(xm, w, y, y32, e0, e1)
        b1.record(s)
        torch.cuda.synchronize()
        if M == 0:
            continue
        rows = ref32 if M == 9 else torch.cat([ref32] * 8, 0)
        assert torch.equal(y32.view(torch.int32), rows.view(torch.int32))
        k_ms, b_ms = e0.elapsed_time(e1), b0.elapsed_time(b1)
        assert 0.0 < k_ms <= b_ms + 1e-3, (M, k_ms, b_ms)


PAIR_CASES = [  # M, K, N0, N1, shared x, with fp32 copies
    (9, 5120, 10240, 17408, True, True),      # the two projections of the short step
    (9, 6144, 4096, 4096, False, True),       # the two halves of the synthetic head
    (1, 5120, 16, 48, False, False),          # fewer column blocks than CUs
    (16, 6144, 4096, 272, True, True),        # a full row tile, uneven split
    (5, 5120, 8192, 16, False, True),         # problem 1 is one block
    (20, 5120, 512, 256, True, True),         # two row tiles: the row-tile kernel, both problems
    (72, 5120, 10240, 17408, True, True),     # batch 8: the two projections in one row-tile launch
    (72, 6144, 4096, 4096, False, True),      # batch 8: the two head halves
    (40, 6144, 4096, 272, False, False),      # three row tiles, uneven
    (9, 1024, 512, 512, False, False),        # other K: one after the other
    (40, 1024, 512, 512, True, False),        # other K, several row tiles: one after the other
]


@pytest.mark.parametrize("case", PAIR_CASES, ids=[str(c) for c in PAIR_CASES])
def test_gemm_pair_gives_the_single_gemm_bits(case):
    """xv_gemm_small_m_pair: each output equals xv_gemm_small_m's bits for it, whether the
    two GEMMs share a launch or not; the launch-recorded interval is positive."""
    from bit_exact_speculative_amd.layer import dev_bf16
    M, K, N0, N1, shared, with32 = case
    rng = np.random.default_rng(M * 31 + N0 + N1 + K)
    xv = _xv()
    x0 = dev_bf16(random_bf16(rng, (M, K)), "cuda")
    x1 = x0 if shared else dev_bf16(random_bf16(rng, (M, K)), "cuda")
    w0 = dev_bf16(random_bf16(rng, (N0, K), 0.02), "cuda")
    w1 = dev_bf16(random_bf16(rng, (N1, K), 0.02), "cuda")
    r0, r0_32 = _gemm_dev(x0, w0)
    r1, r1_32 = _gemm_dev(x1, w1)
    y0 = torch.empty((M, N0), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")
    y0_32 = torch.empty((M, N0), dtype=torch.float32, device="cuda") if with32 else None
    y1_32 = torch.empty((M, N1), dtype=torch.float32, device="cuda") if with32 else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    xv.xv_gemm_small_m_pair(x0, w0, y0, y0_32, x1, w1, y1, y1_32, e0, e1)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16), r0.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), r1.view(torch.int16))
    if with32:
        assert torch.equal(y0_32.view(torch.int32), r0_32.view(torch.int32))
        assert torch.equal(y1_32.view(torch.int32), r1_32.view(torch.int32))
    assert e0.elapsed_time(e1) > 0.0


@pytest.mark.parametrize("M,N,K", [(256, 400, 5120), (300, 10240, 5120), (1000, 272, 6144),
                                   (257, 48, 96), (384, 1040, 544), (2048, 17408, 5120)])
def test_gemm_many_rows_tiled_kernel_rows_equal_k_split(M, N, K):
    """From 256 rows the 128 x 128 tiled kernel runs (prefill); every row must equal the same
    row computed at M <= 16 by the K-split kernels (sampled 9-row slices, including the last
    partial row tile and a column tile cut by N), and sampled columns must match the oracle.
    K = 96 leaves 13 of the 16 ranges empty."""
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(M * 3 + N + K)
    xh = random_bf16(rng, (M, K))
    wh = random_bf16(rng, (N, K), 0.02)
    x = dev_bf16(xh, "cuda"); w = dev_bf16(wh, "cuda")
    y, y32 = _gemm_dev(x, w)
    starts = sorted(set([0, 120, 128, M - 9] + [int(v) for v in rng.integers(0, M - 9, size=4)]))
    for r0 in starts:
        r1 = min(M, r0 + 9)
        ys, ys32 = _gemm_dev(x[r0:r1].contiguous(), w)
        assert torch.equal(ys32.view(torch.int32), y32[r0:r1].view(torch.int32)), r0
        assert torch.equal(ys.view(torch.int16), y[r0:r1].view(torch.int16)), r0
    cols = np.sort(rng.choice(N, size=min(N, 48), replace=False))
    rows = np.sort(rng.choice(M, size=min(M, 64), replace=False))
    ref = oracle.gemm(xh[rows], wh[cols])
    torch.cuda.synchronize()
    assert max_rel(y32.cpu().numpy()[rows][:, cols], ref) <= OUT_MAX_REL


@pytest.mark.parametrize("M,N,K", [(17, 400, 5120), (33, 10240, 5120), (48, 272, 6144), (64, 4096, 6144),
                                   (72, 17408, 5120), (80, 1040, 5120), (72, 4096, 6144)])
def test_gemm_row_tiles_weight_streaming_rows_equal_k_split(M, N, K):
    """2 to 5 row tiles at K = 5120 / 6144 take the weight-streaming row-tile kernel (x from
    L2, W once, 1 to 6 column blocks per workgroup); every row must equal its M <= 16 bits
    and sampled entries the oracle."""
    from bit_exact_speculative_amd.layer import dev_bf16
    rng = np.random.default_rng(M * 5 + N + K)
    xh = random_bf16(rng, (M, K))
    wh = random_bf16(rng, (N, K), 0.02)
    x = dev_bf16(xh, "cuda"); w = dev_bf16(wh, "cuda")
    y, y32 = _gemm_dev(x, w)
    for r0 in sorted(set([0, 16, M - 9] + [int(v) for v in rng.integers(0, M - 9, size=3)])):
        ys, ys32 = _gemm_dev(x[r0:r0 + 9].contiguous(), w)
        assert torch.equal(ys32.view(torch.int32), y32[r0:r0 + 9].view(torch.int32)), r0
        assert torch.equal(ys.view(torch.int16), y[r0:r0 + 9].view(torch.int16)), r0
    cols = np.sort(rng.choice(N, size=min(N, 48), replace=False))
    ref = oracle.gemm(xh, wh[cols])
    torch.cuda.synchronize()
    assert max_rel(y32.cpu().numpy()[:, cols], ref) <= OUT_MAX_REL
