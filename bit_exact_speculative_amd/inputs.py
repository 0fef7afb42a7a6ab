"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the verify step itself: it draws random
numbers, applies the input recipe (L2 normalisation of q and k, the decay and
beta activations, bf16 rounding) and lays the results out.  Both the oracle and
the HIP path consume exactly the arrays produced here.

Workloads (the pages' own prompts are not available; these stand in for them
with the shapes and lengths the recipe card and the post give):

  tiny    one small GDN + attention + GEMM problem the oracle finishes at once
  short   27B-class hybrid layer shapes, batch 1, 640 cached tokens (the card's
          short-prompt bucket), k = 8 drafts -> 9 verify rows
  medium  the same shapes with 2183 cached tokens (a parity prompt length on
          the card), plus a forced-reject case
  batch8  8 requests in flight, cached lengths uniform in 560..740 (the
          repeatability prompts of the post), accepted lengths uniform 0..8
  long    the same shapes with 127735 cached tokens (the card's long prompt)

Draw order.  Two numpy PCG64 streams come from SeedSequence(workload index):
stream A draws items 1-5 and stream B items 6-7 (so skipping the large weight
draws never moves the draft ids).  Every draw is fp32 standard normal unless
stated; the order is fixed, and no capacity (Lmax) or workspace choice moves a
value:
   1. GDN prefix rows (32 tokens): q, k [B][32][Hk][dk]; v [B][32][Hv][dv];
      raw decay [B][32][Hv]; raw beta [B][32][Hv]
   2. GDN verify rows: q, k, v, raw decay, raw beta, same layouts with T rows
   3. attention: cached lengths L0 (batch8 only: integers 560..740), then
      q [B][T][Hq][d], k_new, v_new [B][T][Hkv][d], then for each request b and
      KV head g the cached keys [L0_b][d] followed by the cached values [L0_b][d]
   4. GEMM: x [M][K]; W1 [N1][K] * 0.02; W2 [N2][K] * 0.02
   5. synthetic head: W_head_gdn [NH][Hv*dv] * 0.02; W_head_attn [NH][Hq*d] * 0.02
   6. (stream B) draft ids [B][T] uniform integers in [0, NH)
   7. (stream B) batch8 only: accepted draft counts uniform integers 0..k
   8. (stream C, composed decoding only) token embedding table [NH][K] (bf16
      standard normals), then one root token per request, uniform in [0, NH)

Input recipe: q and k are L2-normalised per (token, head) vector in fp64, then
rounded to fp32 and then to bf16 (round to nearest even); v, x, caches and
weights are rounded fp32 -> bf16; decay a = exp(-softplus(z)) and beta
b = sigmoid(z) are computed in fp64 and rounded to fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

PREFIX_TOKENS = 32
BF16_NAN = 0x7FC0          # quiet NaN bit pattern, used to poison cache slots past the data


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    T: int                       # verify rows = drafts + 1
    # GDN
    Hk: int
    Hv: int
    dk: int
    dv: int
    # attention
    Hq: int
    Hkv: int
    d: int
    L0: Optional[int]            # fixed cached length, or None for a per-request draw
    L0_range: tuple = (0, 0)
    # GEMMs
    K: int = 0
    N1: int = 0
    N2: int = 0
    NH: int = 0                  # synthetic head vocabulary
    accept_draw: bool = False

    @property
    def k_drafts(self) -> int:
        return self.T - 1

    @property
    def M(self) -> int:
        return self.B * self.T


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, T=5, Hk=2, Hv=4, dk=64, dv=64, Hq=4, Hkv=1, d=64,
                     L0=128, K=256, N1=512, N2=512, NH=512),
    "short": Workload("short", 1, B=1, T=9, Hk=16, Hv=48, dk=128, dv=128, Hq=24, Hkv=4, d=256,
                      L0=640, K=5120, N1=10240, N2=17408, NH=4096),
    "medium": Workload("medium", 2, B=1, T=9, Hk=16, Hv=48, dk=128, dv=128, Hq=24, Hkv=4, d=256,
                       L0=2183, K=5120, N1=10240, N2=17408, NH=4096),
    "batch8": Workload("batch8", 3, B=8, T=9, Hk=16, Hv=48, dk=128, dv=128, Hq=24, Hkv=4, d=256,
                       L0=None, L0_range=(560, 740), K=5120, N1=10240, N2=17408, NH=4096,
                       accept_draw=True),
    "long": Workload("long", 4, B=1, T=9, Hk=16, Hv=48, dk=128, dv=128, Hq=24, Hkv=4, d=256,
                     L0=127735, K=5120, N1=10240, N2=17408, NH=4096),
}


# ---------------------------------------------------------------------------
# bf16 helpers (input preparation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, np.uint16)
    _round_into(a.reshape(-1), out.reshape(-1))
    return out


def _round_into(a: np.ndarray, out: np.ndarray) -> None:
    # finite values only: u + 0x7FFF + lsb stays below 2^32 for every finite pattern
    u = a.view(np.uint32)
    t = (u >> 16) & 1
    t += u
    t += 0x7FFF
    t >>= 16
    out[...] = t


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


_CHUNK = 1 << 22


def _normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of scaled fp32 normals, drawn in chunks (the same value stream as one draw)."""
    out = np.empty(shape, np.uint16)
    flat = out.reshape(-1)
    n = flat.size
    buf = np.empty(min(n, _CHUNK), np.float32)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        b = buf[:m]
        rng.standard_normal(out=b, dtype=np.float32)
        if scale != 1.0:
            b *= np.float32(scale)
        _round_into(b, flat[i:i + m])
    return out


def _l2norm_bf16(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))
    return f32_to_bf16_bits((x64 / n).astype(np.float32))


def _decay(z: np.ndarray) -> np.ndarray:
    z64 = z.astype(np.float64)
    softplus = np.logaddexp(0.0, z64)
    return np.exp(-softplus).astype(np.float32)


def _beta(z: np.ndarray) -> np.ndarray:
    z64 = z.astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z64))).astype(np.float32)


def gdn_rows(rng: np.random.Generator, B: int, T: int, Hk: int, Hv: int, dk: int, dv: int):
    """q, k (bf16, L2-normalised), v (bf16), a, b (fp32) for T rows."""
    q = _l2norm_bf16(_normal(rng, (B, T, Hk, dk)))
    k = _l2norm_bf16(_normal(rng, (B, T, Hk, dk)))
    v = _normal_bf16(rng, (B, T, Hv, dv))
    a = _decay(_normal(rng, (B, T, Hv)))
    b = _beta(_normal(rng, (B, T, Hv)))
    return dict(q=q, k=k, v=v, a=a, b=b)


@dataclass
class Inputs:
    wl: Workload
    prefix: dict                 # GDN prefix rows (32 tokens)
    gdn: dict                    # GDN verify rows
    L0: np.ndarray               # int32 [B]
    Lmax: int
    q_attn: np.ndarray           # bf16 [B][T][Hq][d]
    k_new: np.ndarray            # bf16 [B][T][Hkv][d]
    v_new: np.ndarray
    k_cache: np.ndarray          # bf16 [B][Hkv][Lmax][d]
    v_cache: np.ndarray
    x: Optional[np.ndarray] = None     # bf16 [M][K]
    W1: Optional[np.ndarray] = None    # bf16 [N1][K]
    W2: Optional[np.ndarray] = None    # bf16 [N2][K]
    Wh_gdn: Optional[np.ndarray] = None    # bf16 [NH][Hv*dv]
    Wh_attn: Optional[np.ndarray] = None   # bf16 [NH][Hq*d]
    draft: Optional[np.ndarray] = None     # int32 [B][T]
    accepted: Optional[np.ndarray] = None  # int32 [B] (batch8)
    extra: dict = field(default_factory=dict)


def make_inputs(wl: Workload, *, Lmax: Optional[int] = None, pad_value: int = BF16_NAN,
                with_gemm: bool = True, with_head: bool = True) -> Inputs:
    """Generate every input of workload ``wl`` in the documented draw order.

    Lmax: cache capacity (default max(L0) + T).  Cache slots at and past each
    request's cached length are filled with ``pad_value`` (a bf16 NaN by default,
    so that any read of a slot the method must not see shows up in the result).
    with_gemm / with_head=False skip the (large) weight draws; they come last in
    the draw order, so skipping them changes nothing else.
    """
    sa, sb = np.random.SeedSequence(wl.seed).spawn(2)   # stream C is spawned third (composed_inputs)
    rng = np.random.Generator(np.random.PCG64(sa))
    rng_ids = np.random.Generator(np.random.PCG64(sb))
    B, T = wl.B, wl.T
    prefix = gdn_rows(rng, B, PREFIX_TOKENS, wl.Hk, wl.Hv, wl.dk, wl.dv)
    gdn = gdn_rows(rng, B, T, wl.Hk, wl.Hv, wl.dk, wl.dv)
    if wl.L0 is None:
        lo, hi = wl.L0_range
        L0 = rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)
    else:
        L0 = np.full((B,), wl.L0, np.int32)
    if Lmax is None:
        Lmax = int(L0.max()) + T
    if Lmax < int(L0.max()) + T:
        raise ValueError("Lmax too small for L0 + T")
    q_attn = _normal_bf16(rng, (B, T, wl.Hq, wl.d))
    k_new = _normal_bf16(rng, (B, T, wl.Hkv, wl.d))
    v_new = _normal_bf16(rng, (B, T, wl.Hkv, wl.d))
    k_cache = np.full((B, wl.Hkv, Lmax, wl.d), pad_value, np.uint16)
    v_cache = np.full((B, wl.Hkv, Lmax, wl.d), pad_value, np.uint16)
    for bb in range(B):
        n = int(L0[bb])
        for g in range(wl.Hkv):
            k_cache[bb, g, :n] = _normal_bf16(rng, (n, wl.d))
            v_cache[bb, g, :n] = _normal_bf16(rng, (n, wl.d))
    inp = Inputs(wl=wl, prefix=prefix, gdn=gdn, L0=L0, Lmax=Lmax, q_attn=q_attn,
                 k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache)
    inp.draft = rng_ids.integers(0, wl.NH, size=(B, T), dtype=np.int64).astype(np.int32)
    if wl.accept_draw:
        inp.accepted = rng_ids.integers(0, wl.k_drafts + 1, size=B, dtype=np.int64).astype(np.int32)
    if not with_gemm:
        return inp
    inp.x = _normal_bf16(rng, (wl.M, wl.K))
    inp.W1 = _normal_bf16(rng, (wl.N1, wl.K), 0.02)
    inp.W2 = _normal_bf16(rng, (wl.N2, wl.K), 0.02)
    if not with_head:
        return inp
    inp.Wh_gdn = _normal_bf16(rng, (wl.NH, wl.Hv * wl.dv), 0.02)
    inp.Wh_attn = _normal_bf16(rng, (wl.NH, wl.Hq * wl.d), 0.02)
    return inp


def random_bf16(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of scaled standard normals (for ad-hoc test shapes)."""
    return _normal_bf16(rng, shape, scale)


def random_gdn(rng: np.random.Generator, B, T, Hk, Hv, dk, dv):
    """GDN rows with the workload recipe, for ad-hoc test shapes."""
    return gdn_rows(rng, B, T, Hk, Hv, dk, dv)


def composed_inputs(wl: Workload, *, Lmax: Optional[int] = None) -> Inputs:
    """Inputs of composed decoding on the synthetic layer: every array of
    :func:`make_inputs` (the weights, the cached prefix: GDN prefix rows and KV
    cache) plus, from a third stream, the token embedding table (extra["E"],
    bf16 [NH][K]) and the root tokens (extra["root"], int32 [B])."""
    inp = make_inputs(wl, Lmax=Lmax, with_gemm=True, with_head=True)
    sc = np.random.SeedSequence(wl.seed).spawn(3)[2]
    rng = np.random.Generator(np.random.PCG64(sc))
    inp.extra["E"] = _normal_bf16(rng, (wl.NH, wl.K))
    inp.extra["root"] = rng.integers(0, wl.NH, size=wl.B, dtype=np.int64).astype(np.int32)
    return inp
