"""Divergence-margin diagnostic: where does a non-exact verify flip token ids?

The recipe card's receipts report that, without the exactness changes, the
tokens of speculative decoding diverge from plain decoding only where the
top-1 and top-2 logits are close (within 0.25, and within 0.125 for the
backend and max-num-seqs controls).  This module reproduces that measurement
on the synthetic layer:

  * reference: plain greedy decoding through the exact path (every step is
    the decode arithmetic of libxv);
  * the exact speculative run: k drafts verified by libxv (it must never
    diverge);
  * a non-exact speculative run: the same, except that the verify step's two
    projections are computed with a different summation order (torch's fp32
    matrix product of the bf16 inputs, rounded to bf16 like libxv's), the kind
    of M-dependent kernel choice the pages remove.

For every request the first emitted position where a run's id differs from the
reference is a divergence; its margin is the reference logits' top-1 minus
top-2 at that position.  A flip needs the perturbation of the two logits to
exceed the margin, so every margin is at most twice the largest logit change
the non-exact run makes at that position.  Over every position compared (up to
each request's first flip, where both runs have the same token history) the
report gives the margins, the logit changes and the positions at risk (margin
at most twice the change): a flip can only happen at one of those.

Diagnostic only: the non-exact projections use torch and are never part of the
library's path.
"""
from __future__ import annotations

import numpy as np
import torch

from . import inputs as gen
from .decode import Decoder


def _fp32_projections(dec: Decoder, R, tokens):
    """y1, y2 = bf16(x W^T) with torch's fp32 product (a different order than libxv's)."""
    x = R.x.float()
    R.y1.copy_((x @ dec.W1.float().T).to(torch.bfloat16))
    R.y2.copy_((x @ dec.W2.float().T).to(torch.bfloat16))


def _gap(z: np.ndarray) -> float:
    s = np.sort(z.astype(np.float64))
    return float(s[-1] - s[-2])


def divergence_margins(name: str = "batch8", n_tokens: int = 24, k: int = 8, p_wrong: float = 0.3,
                       seeds=(0, 1, 2), S0=None):
    """Runs the three decodings for each draft seed; returns a dict of counts and margins."""
    wl = gen.WORKLOADS[name]
    inp = gen.composed_inputs(wl)
    root = inp.extra["root"]
    Lmax = int(inp.L0.max()) + n_tokens + 2 * k + 4
    ref_dec = Decoder(inp, Lmax, S0=S0)
    snap = ref_dec.snapshot()
    z_ref = []
    ids_ref, _, _ = ref_dec.generate(root, n_tokens + k, logits=z_ref)
    scale = float(np.std(np.stack(z_ref[0][:4])))
    exact_div, rows, seen = 0, [], []
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)

        def drafts(b, pos, kk):
            d = np.array([ids_ref[b, min(pos + i, ids_ref.shape[1] - 1)] for i in range(kk)], np.int32)
            bad = rng.random(kk) < p_wrong
            d[bad] = (d[bad] + 1 + rng.integers(0, wl.NH - 1, int(bad.sum()))) % wl.NH
            return d

        state = rng.bit_generator.state
        ref_dec.restore(snap)
        ids_x, _, _ = ref_dec.generate(root, n_tokens, drafts, k=k)
        exact_div += int(np.sum(np.any(ids_x != ids_ref[:, :n_tokens], axis=1)))
        rng.bit_generator.state = state                 # the same drafts for the non-exact run
        ne = Decoder(inp, Lmax, S0=S0, projections=_fp32_projections)
        ne.restore(snap)
        z_ne = []
        ids_ne, _, _ = ne.generate(root, n_tokens, drafts, k=k, logits=z_ne)
        del ne
        for b in range(wl.B):
            diff = np.nonzero(ids_ne[b] != ids_ref[b, :n_tokens])[0]
            end = int(diff[0]) + 1 if diff.size else n_tokens
            # every position up to and including the first flip: the reference margin and
            # the largest logit change of the non-exact run (same token history until then)
            for p in range(end):
                zr, zn = z_ref[b][p].astype(np.float64), z_ne[b][p].astype(np.float64)
                seen.append((_gap(zr), float(np.max(np.abs(zn - zr)))))
            if diff.size == 0:
                rows.append(None)
                continue
            rows.append({"pos": end - 1, "margin": seen[-1][0], "max_logit_change": seen[-1][1]})
    div = [r for r in rows if r is not None]
    margins = [r["margin"] for r in div]
    mg = np.array([m for m, _ in seen]); dz = np.array([d for _, d in seen])
    return {
        "workload": name, "requests": len(rows), "tokens": n_tokens, "k": k, "p_wrong_draft": p_wrong,
        "exact_spec_diverged": exact_div,
        "nonexact_diverged": len(div),
        "flip_margins": [round(m, 6) for m in margins],
        "positions_compared": int(mg.size),
        "logit_std": round(scale, 6),
        "median_margin": round(float(np.median(mg)), 6),
        "min_margin": round(float(mg.min()), 6),
        "median_logit_change": round(float(np.median(dz)), 8),
        "max_logit_change": round(float(dz.max()), 8),
        "positions_at_risk": int(np.sum(mg <= 2 * dz)),
        "flips_within_perturbation": all(r["margin"] <= 2 * r["max_logit_change"] + 1e-9 for r in div),
    }
