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
  * two non-exact speculative runs, each the exact one with one change in its
    verify steps:
      - fp32_projections: the two projections with a different summation order
        (torch's fp32 matrix product of the bf16 inputs, rounded to bf16 like
        libxv's), the kind of M-dependent kernel choice the pages remove;
      - bf16_beta: the GDN beta rounded to bf16 before the verify recurrence
        while plain decoding keeps it in fp32, the post's first verify bug (a
        verify kernel with another beta precision than decode's).

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


def _bf16_beta(dec: Decoder, R, tokens):
    """beta at bf16 precision (nearest even) in a verify step."""
    if tokens.shape[1] > 1:
        R.b.copy_(R.b.to(torch.bfloat16).float())


VARIANTS = {"fp32_projections": dict(projections=_fp32_projections),
            "bf16_beta": dict(after_split=_bf16_beta)}


def _gap(z: np.ndarray) -> float:
    s = np.sort(z.astype(np.float64))
    return float(s[-1] - s[-2])


def divergence_margins(name: str = "batch8", n_tokens: int = 256, k: int = 8, p_wrong: float = 0.3,
                       seeds=(0, 1, 2), S0=None, variants=("fp32_projections", "bf16_beta")):
    """Per seed (its own root tokens and drafts): plain decoding, the exact speculative run
    and each non-exact variant; returns a dict of counts and margins (per variant)."""
    wl = gen.WORKLOADS[name]
    inp = gen.composed_inputs(wl)
    Lmax = int(inp.L0.max()) + n_tokens + 2 * k + 4
    ref_dec = Decoder(inp, Lmax, S0=S0)
    snap = ref_dec.snapshot()
    exact_div, scale = 0, None
    res = {v: {"rows": [], "seen": []} for v in variants}
    for seed in seeds:
        # each seed decodes from its own root tokens, so the seeds follow distinct trajectories
        root = ((inp.extra["root"].astype(np.int64) + 977 * seed) % wl.NH).astype(np.int32)
        ref_dec.restore(snap)
        z_ref = []
        ids_ref, _, _ = ref_dec.generate(root, n_tokens + k, logits=z_ref)
        if scale is None:
            scale = float(np.std(np.stack(z_ref[0][:4])))
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
        for v in variants:
            rng.bit_generator.state = state             # the same drafts for every run
            ne = Decoder(inp, Lmax, S0=S0, **VARIANTS[v])
            ne.restore(snap)
            z_ne = []
            ids_ne, _, _ = ne.generate(root, n_tokens, drafts, k=k, logits=z_ne)
            del ne
            rows, seen = res[v]["rows"], res[v]["seen"]
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
    out = {"workload": name, "requests": wl.B * len(seeds), "tokens": n_tokens, "k": k,
           "p_wrong_draft": p_wrong, "logit_std": round(scale, 6), "exact_spec_diverged": exact_div,
           "variants": {}}
    for v in variants:
        div = [r for r in res[v]["rows"] if r is not None]
        mg = np.array([m for m, _ in res[v]["seen"]])
        dz = np.array([d for _, d in res[v]["seen"]])
        out["variants"][v] = {
            "diverged": len(div),
            "flip_margins": [round(r["margin"], 6) for r in div],
            "flip_logit_changes": [round(r["max_logit_change"], 6) for r in div],
            # where each flip's margin falls among the margins of every position compared
            "flip_margin_percentiles": [round(float(np.mean(mg < r["margin"])) * 100, 3) for r in div],
            "positions_compared": int(mg.size),
            "median_margin": round(float(np.median(mg)), 6),
            "min_margin": round(float(mg.min()), 6),
            "median_logit_change": round(float(np.median(dz)), 8),
            "max_logit_change": round(float(dz.max()), 8),
            "positions_at_risk": int(np.sum(mg <= 2 * dz)),
            "flips_within_perturbation": bool(div) and all(r["margin"] <= 2 * r["max_logit_change"] + 1e-9
                                                           for r in div),
        }
    return out
