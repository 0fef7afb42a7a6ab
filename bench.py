#!/usr/bin/env python3
"""Benchmark: verified draft tokens per second for one hybrid layer's verify step.

One step is the whole hot path of a speculative step for one layer, on one
stream, with every input already resident in HBM:
    both projection GEMMs in one launch                              xv_gemm_small_m_pair
      (M = B*T rows, K = 5120, N = 10240 and N = 17408)
    the previous step's rollback (its kept rows replayed from its start
      state) and this step's GDN verify, 48 value heads, fp32 state, beside
      attention verify rows + KV append, 24 q / 4 KV heads, d = 256 xv_gdn_attn_verify
    synthetic head over both outputs (2 x 6144 -> 4096) with the   xv_head_greedy_accept
      greedy ids, logprobs, accepted rows and the new KV length
      (one launch at batch 1)
The last step's rollback (xv_rollback_to_prefix) runs inside the timed region
after the last step.
The default workload is batch 1, k = 8 drafts (9 verify rows), 640 cached
tokens.  Steps run as a real decoding loop: each step verifies against the
state and cache the previous step of the same layer left.  Weights, states and
caches are rotated over several layer replicas (about 1.5 GB in all) so that
the 256 MB Infinity Cache cannot serve the weights of the step being timed.

Before timing, verify == sequential decode is checked bit for bit on the same
buffers; a mismatch reports no throughput.  The JSON line carries the roofline
of the dominant kernel (the projection GEMM launch, timed live with HIP events
that the launch records at the kernel's own start and end, on the stream it runs
on) and the fp64 CPU oracle timed on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft tok/s per layer at k=8 (ctx 640/2.2k/128k); HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
GEMM_EVENT_EVERY = 8          # timed steps per live sample of the dominant GEMM
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemm_pair_projections_short_pmc.md")
GEMM_SOURCES = ["bit_exact_speculative_amd/csrc/xv_gemm.hip", "bit_exact_speculative_amd/csrc/xv_common.h"]


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch of the dominant GEMM from the committed rocprofv3 --pmc summary,
    or None when the summary is missing or the kernel source changed since it was taken."""
    try:
        lines = open(PROFILE_PMC).read().splitlines()
    except OSError:
        return None
    vals = {}
    for ln in lines:
        if ln.startswith("- ") and ":" in ln:
            k, v = ln[2:].split(":", 1)
            vals[k.strip()] = v.strip().split()[0] if v.strip() else ""
    if vals.get("kernel source hash") != gemm_source_hash():
        return None
    try:
        return int(float(vals["calibrated HBM bytes per launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_bytes(wl, ctx_mean):
    """Algorithmic bytes per launch of each call of a lazy step (the unit figures of the
    per-kernel roofline): every weight, state, cache and activation byte the call must
    read or write once; the attention workspace round trip is traffic, not counted."""
    B, T, M = wl.B, wl.T, wl.M
    bf, f4 = 2, 4
    proj = (wl.N1 + wl.N2) * wl.K * bf + M * wl.K * bf + M * (wl.N1 + wl.N2) * bf
    state = B * wl.Hv * wl.dk * wl.dv * f4
    gdn_rows = B * T * (2 * wl.Hk * wl.dk * bf + wl.Hv * wl.dv * bf + 2 * wl.Hv * f4) + B * T * wl.Hv * wl.dv * bf
    gdn = 3 * state + gdn_rows          # start state in, kept state and S_T out
    attn = (B * wl.Hkv * (ctx_mean + T) * wl.d * bf * 2 + B * T * wl.Hq * wl.d * bf * 2
            + B * T * wl.Hkv * wl.d * bf * 2)
    kh = wl.Hv * wl.dv
    head = 2 * wl.NH * kh * bf + 2 * M * kh * bf + 2 * M * wl.NH * (bf + f4)
    greedy = 2 * M * wl.NH * f4
    return {"projections": proj, "gdn": gdn, "attention": attn, "gdn_attn": gdn + attn, "head": head,
            "greedy": greedy, "head_greedy": head}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="short", choices=["short", "medium", "long", "batch8"])
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline time budget")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel event pass (per-launch us and GB/s) after the timed steps")
    ap.add_argument("--roofline-samples", type=int, default=32,
                    help="launches of the dominant GEMM timed with launch-recorded events (at least 25)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the medium / batch-8 / long workloads reported beside the headline")
    ap.add_argument("--prefill-only", action="store_true",
                    help="print only the prefill leg (other_workloads.prefill) as one JSON line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--profile", action="store_true",
                    help="only the gate and the timed steps (no full-acceptance pass, no extras, no CPU "
                         "baseline): the launches a profiler run selects by position")
    return ap.parse_args()


def build_layers(wl, Lmax, R, stream, len_bound=True):
    """Inputs for workload wl, R resident layer replicas, and the bit-exact gate
    (verify == sequential decode on the same buffers, every output bit; three lazy steps
    == three steps of verify + rollback, every state, cache and output bit).  len_bound:
    the layers pass their host bound on the lengths to the attention calls (the decode
    sequence of the gate passes none)."""
    import torch
    from bit_exact_speculative_amd import inputs as gen
    from bit_exact_speculative_amd.layer import Layer
    t0 = time.time()
    inp = gen.make_inputs(wl, Lmax=Lmax, pad_value=0)
    print("# inputs generated in %.1f s (workload %s, Lmax %d)" % (time.time() - t0, wl.name, Lmax),
          file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        base = Layer(inp, "cuda")                 # prefix state computed by the GPU path
        base.proj_fp32 = False                    # projections: bf16 outputs only
        base.out_fp32 = False                     # GDN / attention: bf16 outputs only
        base.use_len_bound = len_bound
        gate = base.clone()
        gate.proj_fp32 = True
        gate.verify(rollback=False)
        dec = gate.decode_sequence()
        torch.cuda.synchronize()
        same = lambda a, b: torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                                        b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32))
        exact = (same(gate.o_gdn, dec["o_gdn"]) and same(gate.S_out, dec["S"][-1]) and
                 same(gate.o_attn, dec["o_attn"]) and same(gate.Kc, dec["Kc"]) and
                 same(gate.y1.view(wl.B, wl.T, wl.N1), dec["y1"]) and
                 same(gate.y2_32.view(wl.B, wl.T, wl.N2), dec["y2_32"]) and
                 torch.equal(gate.ids, dec["ids"]))
        del gate, dec
        eager, lazy = base.clone(), base.clone()
        for _ in range(3):
            eager.verify()
            eager.advance()
            lazy.lazy_step()
            exact = exact and same(eager.o_gdn, lazy.o_gdn) and torch.equal(eager.ids, lazy.ids) and \
                same(eager.lp, lazy.lp) and torch.equal(eager.kv_len, lazy.kv_len)
        lazy.settle()
        exact = exact and same(eager.S_in, lazy.S_in) and same(eager.Kc, lazy.Kc)
        del eager, lazy
        layers = [base] + [base.clone() for _ in range(R - 1)]
        torch.cuda.synchronize()
    print("# %d layer replicas resident; verify==decode bit-exact: %s" % (R, exact), file=sys.stderr, flush=True)
    return inp, layers, bool(exact)


def run_steps(layers, stream, steps, warmup, keep_all=False, gemm_events=False):
    """Warmup, then `steps` timed steps rotating over the replicas, bracketed by HIP events
    on the layers' stream.  keep_all: every request keeps all T rows (full acceptance; each
    step rolls back at once); otherwise the greedy acceptance decides and each step's
    rollback runs inside the next step's GDN launch, the last ones before the timed region
    ends.  Returns (ms per step, per-step projection GEMM us, wall s)."""
    import torch
    R = len(layers)
    full = torch.full((layers[0].B,), layers[0].T, dtype=torch.int32, device="cuda") if keep_all else None

    def step(L, ev=None):
        if keep_all:
            L.gemms(ev)
            L.gdn()
            L.attn()
            L.head()
            L.rollback(full)
            L.advance()
        else:
            L.lazy_step(ev)                       # ev: recorded at the GEMM's own start and end

    with torch.cuda.stream(stream):
        for s in range(warmup):
            step(layers[s % R])
        torch.cuda.synchronize()
        # launch-recorded events on every GEMM_EVENT_EVERY-th step's projection launch: a sample of
        # the timed launches, so that the events' own cost (~4.5 us per event-carrying step)
        # stays out of the step time
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               if gemm_events and s % GEMM_EVENT_EVERY == 0 else None for s in range(steps)]
        for ev in evs:                            # create the events before the timed region
            if ev is not None:
                ev[0].record(stream)
                ev[1].record(stream)
        e_start = torch.cuda.Event(enable_timing=True)
        e_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e_start.record(stream)
        for s in range(steps):
            step(layers[(warmup + s) % R], evs[s])
        for L in layers:
            L.settle()
        e_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    ms = e_start.elapsed_time(e_end) / steps
    gemm_us = [ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs if ev is not None]
    return ms, gemm_us, wall


def lmax_for(wl, steps_per_replica_n1, steps_per_replica_full):
    """Cache capacity for a run: one kept row per greedy step, T per full-acceptance step."""
    L0max = wl.L0 if wl.L0 is not None else wl.L0_range[1]
    return L0max + max(wl.T * (steps_per_replica_n1 + 4), wl.T * (steps_per_replica_full + 4))


def extra_workload(name, stream, steps, warmup, R, capacity=None, len_bound=True):
    """Verified draft tok/s of another workload (bit-exact gate included); capacity: the
    cache's position count (default: the steps' need); len_bound: as build_layers."""
    import torch
    from bit_exact_speculative_amd import inputs as gen
    wl = gen.WORKLOADS[name]
    per = (steps + warmup + R - 1) // R
    Lmax = lmax_for(wl, per, 0) if capacity is None else max(capacity, lmax_for(wl, per, 0))
    _, layers, exact = build_layers(wl, Lmax, R, stream, len_bound)
    ms, _, _ = run_steps(layers, stream, steps, warmup)
    ctx = wl.L0 if wl.L0 is not None else "%d-%d" % wl.L0_range
    res = {"ctx": ctx, "batch": wl.B, "tok_s": round(wl.B * wl.k_drafts / (ms * 1e-3), 1) if exact else None,
           "ms_per_step": round(ms, 5), "bit_exact_verify_equals_decode": exact, "steps": steps,
           "layer_replicas": R, "cache_positions": Lmax}
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def prefill_workload(stream, P=8192, check=256, reps=2, chunk=8192, tail=16):
    """Prefill of a P-token prompt (one chunk of 8192) on the synthetic layer, short workload
    shapes, appended to its 640 cached tokens: embedding, both projections and the split over
    all rows, GDN and attention over all rows (decode arithmetic per row), the head and the
    first token.
    Gated, bit for bit, on (1) the first `check` prompt tokens giving the state, cache, first
    token and logprob of one-token decoding, and (2) the whole prompt: its prefill against the
    prefill of all but its last `tail` tokens followed by `tail` one-token steps (the final
    state, the cache rows of the whole prompt, the first token and its logprob)."""
    import numpy as np
    import torch
    from bit_exact_speculative_amd import inputs as gen
    from bit_exact_speculative_amd.decode import Decoder
    wl = gen.WORKLOADS["short"]
    inp = gen.composed_inputs(wl)
    Lmax = int(inp.L0.max()) + P + 32
    prompt = np.random.default_rng(777).integers(0, wl.NH, size=(wl.B, P)).astype(np.int32)
    with torch.cuda.stream(stream):
        dec = Decoder(inp, Lmax, stream=stream)
        snap = dec.snapshot()
        id_a, lp_a = dec.prefill(prompt[:, :check])
        got = (dec.S.clone(), dec.Kc.clone(), dec.kv_len.clone(), id_a.clone(), lp_a.clone())
        dec.restore(snap)
        for t in range(check):
            R = dec.step(torch.from_numpy(prompt[:, t:t + 1].copy()).to("cuda"))
        want = (dec.S, dec.Kc, dec.kv_len, R.ids[:, 0], R.lp[:, 0])
        torch.cuda.synchronize()
        same = lambda a, b: torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                                        b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32))
        exact = all(same(a, b) for a, b in zip(got, want))
        # the whole prompt: prefill of P - tail tokens then tail one-token steps, against the
        # prefill of all P
        dec.restore(snap)
        dec.prefill(prompt[:, :P - tail], chunk=chunk)
        for t in range(P - tail, P):
            R = dec.step(torch.from_numpy(prompt[:, t:t + 1].copy()).to("cuda"))
        m = int(inp.L0.max()) + P
        want = (dec.S.clone(), dec.Kc[:, :, :m].clone(), dec.kv_len.clone(), R.ids[:, 0].clone(),
                R.lp[:, 0].clone())
        dec.restore(snap)
        id_f, lp_f = dec.prefill(prompt, chunk=chunk)
        got = (dec.S, dec.Kc[:, :, :m], dec.kv_len, id_f, lp_f)
        torch.cuda.synchronize()
        exact_full = all(same(a, b) for a, b in zip(got, want))
        del want, got
        exact = exact and exact_full
        best = None
        for _ in range(reps + 1):                    # the first pass warms up
            dec.restore(snap)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dec.prefill(prompt, chunk=chunk)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None or ms < best else best
    res = {"prompt_tokens": P, "ctx_before": int(inp.L0[0]), "batch": wl.B, "chunk": chunk,
           "bit_exact_prefill_equals_decode": bool(exact), "check_tokens": check,
           "check_whole_prompt": "prefill of %d tokens == prefill of %d + %d one-token steps" % (P, P - tail, tail),
           "tok_s": round(wl.B * P / (best * 1e-3), 1) if exact else None, "ms": round(best, 3),
           "note": "one layer; every prompt row kept; first token formed"}
    del dec
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def composed_workload(stream, n_tokens=48, k=8, p_wrong=0.2, reps=3):
    """Greedy decoding on the synthetic layer, short workload shapes: every step embeds its
    tokens, runs both projections, the split, GDN, attention, the head, logprobs, acceptance
    and rollback.  Emitted tok/s with k drafts (each draft independently wrong with
    probability p_wrong, else the plain-decoding token) and without drafts.  Each run is
    decoded once with host readback, recording every step's input tokens, and gated on the
    same ids and logprobs with and without drafts; the timed region then replays the
    recorded steps from the same start state, so it holds the decoding kernels only."""
    import numpy as np
    import torch
    from bit_exact_speculative_amd import inputs as gen
    from bit_exact_speculative_amd.decode import Decoder
    wl = gen.WORKLOADS["short"]
    inp = gen.composed_inputs(wl)
    root = inp.extra["root"]
    Lmax = int(inp.L0.max()) + n_tokens + 2 * k + 4
    with torch.cuda.stream(stream):
        dec = Decoder(inp, Lmax, stream=stream)
        snap = dec.snapshot()
        rec_plain, rec_spec = [], []
        ids_p, lp_p, _ = dec.generate(root, n_tokens + k, record=rec_plain)
        rng = np.random.default_rng(12345)

        def drafts(b, pos, kk):
            d = np.array([ids_p[b, min(pos + i, ids_p.shape[1] - 1)] for i in range(kk)], np.int32)
            bad = rng.random(kk) < p_wrong
            d[bad] = (d[bad] + 1 + rng.integers(0, wl.NH - 1, int(bad.sum()))) % wl.NH
            return d

        dec.restore(snap)
        ids_s, lp_s, keeps = dec.generate(root, n_tokens, drafts, k=k, record=rec_spec)
        exact = bool(np.array_equal(ids_p[:, :n_tokens], ids_s) and
                     np.array_equal(lp_p[:, :n_tokens].view(np.int32), lp_s.view(np.int32)))
        emitted_spec = int(sum(int(x.sum()) for x in keeps))
        rec_plain = rec_plain[:n_tokens]

        def replay(records):
            toks = torch.from_numpy(np.stack(records)).to("cuda")
            best = None
            for _ in range(reps + 1):                 # the first pass warms up
                dec.restore(snap)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for s in range(toks.shape[0]):
                    dec.step(toks[s])
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1)
                best = ms if best is None or ms < best else best
            return best

        ms_plain = replay(rec_plain)
        ms_spec = replay(rec_spec)
        emitted_plain = wl.B * len(rec_plain)
    res = {"ctx": int(inp.L0[0]), "batch": wl.B, "k": k, "p_wrong_draft": p_wrong,
           "bit_exact_spec_equals_plain": exact,
           "spec_tok_s": round(emitted_spec / (ms_spec * 1e-3), 1) if exact else None,
           "plain_tok_s": round(emitted_plain / (ms_plain * 1e-3), 1),
           "spec_steps": len(rec_spec), "spec_tokens": emitted_spec,
           "tokens_per_spec_step": round(emitted_spec / len(rec_spec) / wl.B, 2),
           "ms_per_spec_step": round(ms_spec / len(rec_spec), 5),
           "ms_per_plain_step": round(ms_plain / len(rec_plain), 5),
           "note": "one layer's weights and embedding table (425 MB) resident; replay of recorded steps"}
    del dec
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU (requests would shard across GPUs with no exchange); "
              "--gpus %d is not supported (use --gpus 1)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from bit_exact_speculative_amd import inputs as gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.prefill_only:                         # one leg, for profiling the prefill path
        print(json.dumps(prefill_workload(torch.cuda.Stream())), flush=True)
        return
    wl = gen.WORKLOADS[args.workload]
    R = max(1, args.replicas)
    full_steps, full_warmup = max(args.steps // 2, 1), max(args.warmup // 2, 1)
    n_extra = max(args.roofline_samples, 25, 0 if args.no_breakdown else 50)     # longest post-timing pass
    Lmax = lmax_for(wl, max(args.warmup + args.steps, n_extra + args.warmup) // R + 1,
                    (full_warmup + full_steps + R - 1) // R)
    stream = torch.cuda.Stream()
    inp, layers, exact = build_layers(wl, Lmax, R, stream)

    # headline: greedy acceptance on the synthetic head (mostly the root row kept, so the
    # rollback recomputes the state), live HIP events on the dominant GEMM's launch
    ms_per_step, gemm_us, wall = run_steps(layers, stream, args.steps, args.warmup, gemm_events=True)
    n_keep = [int(L.n_keep.sum().item()) for L in layers]

    # more launch-recorded samples of the dominant GEMM (steps exactly like the timed ones,
    # after the timed region so that the events' own cost stays out of the step time)
    post_us = []
    for L in layers:                              # back to the pre-verify caches and lengths
        L.settle()
        L.reset()
    with torch.cuda.stream(stream):
        n_post = max(args.roofline_samples - len(gemm_us), 25 - len(gemm_us), 0)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_post)]
        for s_ in range(n_post):
            layers[(args.warmup + args.steps + s_) % R].lazy_step(evs[s_])
        torch.cuda.synchronize()
        post_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    all_gemm_us = gemm_us + post_us

    # the streaming-read ceiling of the same bytes: both projection weights of a replica last
    # read R steps ago, read once by xv_stream_read (launch-recorded events)
    from bit_exact_speculative_amd import xv
    read_us = []
    with torch.cuda.stream(stream):
        sink = torch.empty((4096,), dtype=torch.int32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(12)]
        for i, (e0, e1) in enumerate(evs):
            L = layers[i % R]
            xv.xv_stream_read(L.W1, L.W2, sink, e0, e1)
        torch.cuda.synchronize()
        read_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
    read_bytes = (wl.N1 + wl.N2) * wl.K * 2
    read_med_us = float(np.median(read_us[R:])) if len(read_us) > R else float(np.median(read_us))

    # per-call time of a lazy step: events between the calls of 50 steps queued back to back
    breakdown = None
    if not args.no_breakdown:
        names = ["projections", "gdn_attn", "head_greedy"]
        acc = {k: [] for k in names}
        nb = 50
        for L in layers:
            L.settle()
            L.reset()
        with torch.cuda.stream(stream):
            rec = []
            for s_ in range(nb):
                L = layers[s_ % R]
                fns = [L.gemms, L.gdn_attn_lazy, lambda: L.head_greedy(count_kv=True)]
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
                ev[0].record(stream)
                for i, f in enumerate(fns):
                    f()
                    ev[i + 1].record(stream)
                rec.append(ev)
            torch.cuda.synchronize()
            for ev in rec[2:]:
                for i, k in enumerate(names):
                    acc[k].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
        ctx_mean = float(np.mean(inp.L0))
        kb = kernel_bytes(wl, ctx_mean)
        breakdown = {}
        for k in names:
            us = float(np.median(acc[k]))
            breakdown[k] = {"us": round(us, 2), "algorithmic_bytes": int(kb[k]),
                            "GB_s": round(kb[k] / (us * 1e-6) / 1e9, 1)}
        breakdown["gdn_attn"]["parts_bytes"] = {"gdn": int(kb["gdn"]), "attention": int(kb["attention"])}
        breakdown["note"] = ("median over 48 steps of events recorded between the calls of a lazy step "
                             "(gdn_attn: GDN verify after the previous rollback, attention partials with the "
                             "KV append and the combine); bytes: every weight, state, cache and activation "
                             "byte the call must move once")

    # the same workload with every draft accepted (rollback keeps S_T as is)
    ms_full = None
    if not args.profile:
        for L in layers:
            L.settle()
            L.reset()
        ms_full, _, _ = run_steps(layers, stream, full_steps, full_warmup, keep_all=True)

    if args.calib_copy_mib > 0:
        with torch.cuda.stream(stream):
            src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

    extras = None
    if not args.no_extras and not args.profile and args.workload == "short":
        del layers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        extras = {}
        for name, steps, warmup, reps in (("medium", 100, 10, 4), ("batch8", 100, 10, 4), ("long", 40, 4, 4)):
            try:
                extras[name] = extra_workload(name, stream, steps, warmup, reps)
            except Exception as exc:                  # reported, never hides the headline line
                extras[name] = {"error": "%s: %s" % (type(exc).__name__, exc)}
        # the launch command's context length, short rows: with the host's bound on the lengths
        # (the launch sized for the rows) and without it (sized for the capacity)
        for key, lb, note in (
                ("short_capacity_262144", True,
                 "the short workload in caches of 262,144 positions; the layer passes its host bound on the "
                 "lengths (max L0 + T per step), so the attention launch is sized for the rows: the per-tile "
                 "split, in one launch with GDN"),
                ("short_capacity_262144_no_bound", False,
                 "as short_capacity_262144 without the bound: the launch is sized for the capacity (the "
                 "streaming kernel and the long-row combine); the same bits")):
            try:
                extras[key] = extra_workload("short", stream, 100, 10, 4, capacity=262144, len_bound=lb)
                extras[key]["note"] = note
            except Exception as exc:
                extras[key] = {"error": "%s: %s" % (type(exc).__name__, exc)}
        try:
            extras["composed"] = composed_workload(stream)
        except Exception as exc:
            extras["composed"] = {"error": "%s: %s" % (type(exc).__name__, exc)}
        try:
            extras["prefill"] = prefill_workload(stream)
        except Exception as exc:
            extras["prefill"] = {"error": "%s: %s" % (type(exc).__name__, exc)}
        try:                                      # the pages' 128k prompt, one layer
            extras["prefill_128k"] = prefill_workload(stream, P=127735, reps=1)
        except Exception as exc:
            extras["prefill_128k"] = {"error": "%s: %s" % (type(exc).__name__, exc)}
        try:
            from bit_exact_speculative_amd.diagnose import divergence_margins
            with torch.cuda.stream(stream):
                extras["divergence"] = divergence_margins("batch8", n_tokens=512, k=8, p_wrong=0.3,
                                                          seeds=(0, 1, 2, 3, 4, 5))
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        except Exception as exc:
            extras["divergence"] = {"error": "%s: %s" % (type(exc).__name__, exc)}

    # algorithmic bytes of the dominant kernel (both weights + activations in once + bf16 out)
    M = wl.M
    gemm_bytes = (wl.N1 + wl.N2) * wl.K * 2 + M * wl.K * 2 + M * (wl.N1 + wl.N2) * 2
    gemm_avg_us = float(np.mean(all_gemm_us))
    achieved = gemm_bytes / (gemm_avg_us * 1e-6) / 1e9
    value = wl.B * wl.k_drafts / (ms_per_step * 1e-3) if exact else None

    cpu = None
    if not args.no_cpu_baseline and not args.profile:
        cpu = cpu_baseline(inp, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 1) if value is not None else None,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "%s: batch %d, k=%d drafts (%d verify rows), ctx %s, hidden %d, GDN %d/%d heads "
                        "d=%d fp32 state, attention %d/%d heads d=%d bf16 KV, GEMMs %dx%dx%d and %dx%dx%d, "
                        "head 2x%d->%d" % (wl.name, wl.B, wl.k_drafts, wl.T,
                                           wl.L0 if wl.L0 is not None else "%d-%d" % wl.L0_range,
                                           wl.K, wl.Hk, wl.Hv, wl.dk, wl.Hq, wl.Hkv, wl.d,
                                           M, wl.K, wl.N1, M, wl.K, wl.N2, wl.Hv * wl.dv, wl.NH),
            "global_batch": wl.B,
            "verify_rows": wl.T,
            "layer_replicas": R,
            "bit_exact_verify_equals_decode": bool(exact),
            "rows_kept_per_step": round(float(np.mean(n_keep)) / wl.B, 2) if n_keep else None,
            "verify_rows_per_s": round(wl.B * wl.T / (ms_per_step * 1e-3), 1),
            "compute": "bf16 x bf16 -> fp32 MFMA GEMMs and attention; fp32 GDN state and VALU",
        },
        "full_accept": None if ms_full is None else {
            "value": round(wl.B * wl.k_drafts / (ms_full * 1e-3), 1) if exact else None,
            "ms_per_step": round(ms_full, 5),
            "steps": full_steps,
            "note": "same workload, every request keeps all %d rows (no state recompute)" % wl.T,
        },
        "roofline": {
            "kernel": "xv_gemm_small_m_pair, LDS-staged two-GEMM launch (M=%d, K=%d, N=%d+%d)" % (
                M, wl.K, wl.N1, wl.N2),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(),
            "algorithmic_bytes": gemm_bytes,
            "avg_us": round(gemm_avg_us, 3),
            "samples": len(all_gemm_us),
            "samples_in_timed_region": len(gemm_us),
            "avg_us_in_timed_region": round(float(np.mean(gemm_us)), 3) if gemm_us else None,
            "read_ceiling": {
                "kernel": "xv_stream_read of the same two weight buffers, read R steps after their last use",
                "bytes": read_bytes,
                "us": round(read_med_us, 3),
                "GB_s": round(read_bytes / (read_med_us * 1e-6) / 1e9, 1),
                "achieved_over_ceiling": round(achieved * read_med_us * 1e-6 * 1e9 / read_bytes, 4),
            },
        },
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
    }
    if extras is not None:
        out["other_workloads"] = extras
    if breakdown is not None:
        out["per_call"] = breakdown
    print(json.dumps(out), flush=True)


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle running the same step (both GEMMs, GDN, attention, head, greedy,
    rollback) on the host, repeated until the time budget is spent; tok/s at the same unit."""
    import numpy as np
    import oracle
    wl = inp.wl
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    os.environ.setdefault("OMP_NUM_THREADS", str(threads))
    p = inp.prefix
    _, S_pre, _ = oracle.gdn(p["q"], p["k"], p["v"], p["a"], p["b"],
                             np.zeros((wl.B, wl.Hv, wl.dk, wl.dv), np.float32))
    S0 = S_pre.astype(np.float32)
    g = inp.gdn
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        oracle.gemm(inp.x, inp.W1)
        oracle.gemm(inp.x, inp.W2)
        o_g, _, _ = oracle.gdn(g["q"], g["k"], g["v"], g["a"], g["b"], S0)
        o_a = oracle.attn(inp.q_attn, inp.k_new, inp.v_new, inp.k_cache, inp.v_cache, inp.L0,
                          1.0 / np.sqrt(wl.d))
        from bit_exact_speculative_amd.inputs import f32_to_bf16_bits
        fg = f32_to_bf16_bits(o_g.astype(np.float32)).reshape(wl.M, -1)
        fa = f32_to_bf16_bits(o_a.astype(np.float32)).reshape(wl.M, -1)
        logits = oracle.gemm(fg, inp.Wh_gdn) + oracle.gemm(fa, inp.Wh_attn)
        _, n_keep = oracle.greedy(logits.reshape(wl.B, wl.T, wl.NH), inp.draft)
        oracle.rollback(g["k"], g["v"], g["a"], g["b"], S0, inp.L0, n_keep)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() >= t_end:
            break
    t = float(np.median(times))
    return {"value": round(wl.B * wl.k_drafts / t, 3), "unit": "tok/s", "cores": threads,
            "kind": "oracle",
            "sample": "the full %s step (all rows of every kernel), fp64 C oracle with OpenMP, "
                      "median of %d runs of %.2f s" % (wl.name, len(times), t),
            "verify_rows_per_s": round(wl.B * wl.T / t, 3),
            "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count()}


if __name__ == "__main__":
    main()
