"""Helpers shared by the GPU tests (comparison rules and cached workloads)."""
import functools

import numpy as np
import torch

import oracle
from bit_exact_speculative_amd import inputs as gen

# Tolerances of the oracle comparison (fp64 oracle vs fp32 GPU):
STATE_REL_L2 = 1e-4      # ||S_gpu - S_ref||_F / ||S_ref||_F
OUT_MAX_REL = 2e-3       # max_i |g_i - r_i| / max(|r_i|, FLOOR * RMS(r)), outputs before bf16 rounding
OUT_FLOOR = 1e-2         # elements below 1% of the tensor's RMS are judged against that floor
OUT_REL_L2 = 1e-4        # normwise check of the same outputs


def bits(t: torch.Tensor) -> torch.Tensor:
    """Bit view of a tensor for exact comparison."""
    if t.dtype in (torch.float32,):
        return t.contiguous().view(torch.int32)
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.contiguous().view(torch.int16)
    return t


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and torch.equal(bits(a), bits(b))


def max_rel(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    floor = OUT_FLOOR * np.sqrt(np.mean(r * r))
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor)))


def rel_l2(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((g - r).ravel()) / np.linalg.norm(r.ravel()))


def prefix_state(inp) -> np.ndarray:
    """fp32 GDN state after the 32-token prefix from zero, computed by the oracle (fp64 -> fp32)."""
    p = inp.prefix
    wl = inp.wl
    _, S, _ = oracle.gdn(p["q"], p["k"], p["v"], p["a"], p["b"],
                         np.zeros((wl.B, wl.Hv, wl.dk, wl.dv), np.float32))
    return S.astype(np.float32)


@functools.lru_cache(maxsize=None)
def workload(name: str, gemm: bool = True, head: bool = True):
    wl = gen.WORKLOADS[name]
    inp = gen.make_inputs(wl, with_gemm=gemm, with_head=head)
    return inp, prefix_state(inp)
