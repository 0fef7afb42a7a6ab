"""Greedy decoding of one synthetic hybrid layer on the GPU, with or without
speculative verification, built from libxv calls only.

A decoding step consumes tokens[b] = [root, draft_1 .. draft_k] (k = 0: plain
decoding) and runs, on one stream:

  xv_embed_rows         x = E[tokens]
  xv_gemm_small_m_pair  y1 = x W1^T, y2 = x W2^T (one launch)
  xv_split_projections  GDN q, k (L2-normalised), v, decay, beta; attention q, k, v
  xv_gdn_verify         GDN rows, S_in -> S_T
  xv_attn_verify_rows   attention rows, KV append (with the GDN rows: xv_gdn_attn_verify)
  xv_head_greedy_accept head logits from o_gdn and o_attn, ids, logprobs, accepted rows
  xv_rollback_to_prefix state and KV length of the kept rows

and emits ids[b][0 .. n_keep[b]-1]; the last one is the next root.  With
lazy=True (the default) the rollback is folded into the next step: the greedy
kernel adds n_keep to the KV length, and the next step's xv_gdn_verify_after
replays the kept rows from the previous start state (or takes S_T when every
row was kept) before its own rows, in one xv_gdn_attn_verify call with the
attention rows; the state of the kept rows is materialised only when asked for
(settle()).  Both ways give the same bits.  The post's
claim (first paragraph; the paragraph on the two verify changes) is that the
emitted ids and logprobs do not depend on k or on the drafts; the tests check
that bit for bit.  Torch provides device memory and the stream only.
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np
import torch

from . import xv
from .inputs import Inputs, PREFIX_TOKENS


def _bf16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def prefix_state(inp: Inputs, device, stream=None) -> torch.Tensor:
    """The GDN state after the workload's 32 prefix tokens from a zero state (GPU path)."""
    wl, p = inp.wl, inp.prefix
    B = wl.B
    S = torch.zeros((B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=device)
    S2 = torch.empty_like(S)
    t0 = 0
    while t0 < PREFIX_TOKENS:
        tt = min(16, PREFIX_TOKENS - t0)
        sl = slice(t0, t0 + tt)
        o = torch.empty((B, tt, wl.Hv, wl.dv), dtype=torch.bfloat16, device=device)
        xv.xv_gdn_verify(_bf16(p["q"][:, sl], device), _bf16(p["k"][:, sl], device),
                         _bf16(p["v"][:, sl], device),
                         torch.from_numpy(np.ascontiguousarray(p["a"][:, sl])).to(device),
                         torch.from_numpy(np.ascontiguousarray(p["b"][:, sl])).to(device),
                         S, S2, o, None, stream=stream)
        S, S2 = S2, S
        t0 += tt
    return S


class _Rows:
    """Device buffers for steps of T rows per request."""

    def __init__(self, wl, T: int, Lmax: int, device):
        B, M = wl.B, wl.B * T
        e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=device)
        f = lambda *s: torch.empty(s, dtype=torch.float32, device=device)
        self.T = T
        self.tokens = torch.empty((B, T), dtype=torch.int32, device=device)
        self.x = e(M, wl.K)
        self.y1, self.y2 = e(M, wl.N1), e(M, wl.N2)
        self.q, self.k = e(B, T, wl.Hk, wl.dk), e(B, T, wl.Hk, wl.dk)
        self.v = e(B, T, wl.Hv, wl.dv)
        self.a, self.b = f(B, T, wl.Hv), f(B, T, wl.Hv)
        self.qa = e(B, T, wl.Hq, wl.d)
        self.kn, self.vn = e(B, T, wl.Hkv, wl.d), e(B, T, wl.Hkv, wl.d)
        self.o_gdn, self.o_attn = e(B, T, wl.Hv, wl.dv), e(B, T, wl.Hq, wl.d)
        self.lg, self.la = e(M, wl.NH), e(M, wl.NH)
        self.lg32, self.la32 = f(M, wl.NH), f(M, wl.NH)
        self.ids = torch.empty((B, T), dtype=torch.int32, device=device)
        self.lp = f(B, T)
        self.n_keep = torch.empty((B,), dtype=torch.int32, device=device)
        self.ws = xv.xv_attn_workspace(B, T, wl.Hq, wl.d, Lmax, device)


class Decoder:
    """The synthetic layer's weights and decoding state on one device.

    inp: :func:`inputs.composed_inputs` (weights, embedding table, cached prefix).
    S0: optional fp32 [B][Hv][dk][dv] start state (default: the prefix on the GPU).
    Lmax: KV capacity (at least the cached length + every token decoded + one step).
    """

    def __init__(self, inp: Inputs, Lmax: int, device="cuda", S0: Optional[np.ndarray] = None, stream=None,
                 projections: Optional[Callable] = None, lazy: bool = True, after_split: Optional[Callable] = None):
        """projections(decoder, rows, tokens): an alternative that fills rows.y1 and rows.y2
        from rows.x (for diagnostics of non-exact variants); None = xv_gemm_small_m_pair.
        after_split(decoder, rows, tokens): diagnostics only, called after the split (it may
        change the operands of GDN and attention in place, as a non-exact variant would).
        lazy: fold each step's rollback into the next step's GDN launch."""
        wl = inp.wl
        self.wl, self.device, self.stream = wl, device, stream
        self.projections = projections
        self.after_split = after_split
        if Lmax < inp.k_cache.shape[2]:
            raise ValueError("Lmax below the inputs' cache capacity")
        self.E = _bf16(inp.extra["E"], device)
        self.W1, self.W2 = _bf16(inp.W1, device), _bf16(inp.W2, device)
        self.Wh_g, self.Wh_a = _bf16(inp.Wh_gdn, device), _bf16(inp.Wh_attn, device)
        B = wl.B
        self.Kc = torch.zeros((B, wl.Hkv, Lmax, wl.d), dtype=torch.bfloat16, device=device)
        self.Vc = torch.zeros_like(self.Kc)
        L = inp.k_cache.shape[2]
        self.Kc[:, :, :L] = _bf16(inp.k_cache, device)
        self.Vc[:, :, :L] = _bf16(inp.v_cache, device)
        self.kv_len = torch.from_numpy(inp.L0.astype(np.int32)).to(device)
        # host upper bound on max(kv_len) (a step adds at most T rows, a prefill P): the
        # attention launch is sized for _kv_hi + T positions, not the capacity (the same bits)
        self._kv_hi = int(inp.L0.max()) if B else 0
        if S0 is None:
            self._S = prefix_state(inp, device, stream)
        else:
            self._S = torch.from_numpy(np.ascontiguousarray(S0, dtype=np.float32)).to(device)
        self._S2 = torch.empty_like(self._S)
        self.lazy = lazy
        # lazy mode: (rows of the last step, its start state, its S_T), and two free states;
        # while a step is pending, _S and _S2 are its start state and its S_T
        self._pending = None
        self._free = (torch.empty_like(self._S), torch.empty_like(self._S)) if lazy else None
        self._kv_scratch = torch.zeros_like(self.kv_len)
        self._slot = 0
        self.Lmax = Lmax
        self.scale = 1.0 / float(wl.d) ** 0.5
        self._rows = {}
        self._hg = None

    def _hg_ws(self, B: int, T: int) -> torch.Tensor:
        """The head + greedy call's workspace (zero at allocation; each call leaves it so)."""
        n = xv.xv_head_greedy_workspace_bytes(B, T, self.wl.NH)
        if getattr(self, "_hg", None) is None or self._hg.numel() < n:
            self._hg = torch.zeros((n,), dtype=torch.uint8, device=self.device)
        return self._hg

    def rows(self, T: int, slot: int = 0) -> _Rows:
        key = (T, slot)
        if key not in self._rows:
            self._rows[key] = _Rows(self.wl, T, self.Lmax, self.device)
        return self._rows[key]

    @property
    def S(self) -> torch.Tensor:
        """The GDN state after every kept row (settles a pending rollback)."""
        self.settle()
        return self._S

    def settle(self):
        """Lazy mode: run the last step's rollback now (the KV length was already updated)."""
        if self._pending is None:
            return
        Rp, P, Q = self._pending
        xv.xv_rollback_to_prefix(Rp.k, Rp.v, Rp.a, Rp.b, P, Q, self._kv_scratch, Rp.n_keep,
                                 stream=self.stream)
        self._S, self._S2 = Q, P
        self._pending = None

    def step(self, tokens: torch.Tensor) -> _Rows:
        """One decoding step over tokens, a contiguous int32 [B][T] device tensor (read in
        place); returns the row buffers, whose ids, lp and n_keep hold the step's results.
        The state advances to the kept rows."""
        wl, st = self.wl, self.stream
        B, T = tokens.shape
        R = self.rows(T, self._slot)
        if self.lazy:
            self._slot ^= 1                  # the previous step's rows stay intact for the replay
        M = B * T
        xv.xv_embed_rows(self.E, tokens, R.x, stream=st)
        if self.projections is None:
            xv.xv_gemm_small_m_pair(R.x, self.W1, R.y1, None, R.x, self.W2, R.y2, None, stream=st)
        else:
            self.projections(self, R, tokens)
        xv.xv_split_projections(R.y1, R.y2, R.q, R.k, R.v, R.a, R.b, R.qa, R.kn, R.vn, stream=st)
        if self.after_split is not None:
            self.after_split(self, R, tokens)
        lb = min(self._kv_hi + T, self.Lmax)
        if not self.lazy:
            xv.xv_gdn_verify(R.q, R.k, R.v, R.a, R.b, self._S, self._S2, R.o_gdn, None, stream=st)
            xv.xv_attn_verify_rows(R.qa, R.kn, R.vn, self.Kc, self.Vc, self.kv_len, R.o_attn, None, R.ws,
                                   self.scale, len_bound=lb, stream=st)
        else:
            # GDN (after the pending step's rollback) and attention in one call
            if self._pending is None:
                out, prev = self._S2, None
            else:
                Rp, P, Q = self._pending
                K, O = self._free
                out, prev = O, (Rp.k, Rp.v, Rp.a, Rp.b, Rp.n_keep, Q, K)
            xv.xv_gdn_attn_verify(R.q, R.k, R.v, R.a, R.b, self._S, out, R.o_gdn, R.qa, R.kn, R.vn,
                                  self.Kc, self.Vc, self.kv_len, R.o_attn, R.ws, self.scale, prev=prev,
                                  len_bound=lb, stream=st)
            if self._pending is None:
                self._pending = (R, self._S, self._S2)
            else:
                self._pending, self._free = (R, K, O), (P, Q)
                self._S, self._S2 = K, O     # the pending step's start state and S_T
        xv.xv_head_greedy_accept(R.o_gdn.view(M, wl.Hv * wl.dv), self.Wh_g, R.lg, R.lg32,
                                 R.o_attn.view(M, wl.Hq * wl.d), self.Wh_a, R.la, R.la32, tokens, R.ids,
                                 R.n_keep, self._hg_ws(B, T), logprob=R.lp,
                                 kv_len=self.kv_len if self.lazy else None, stream=st)
        if not self.lazy:
            xv.xv_rollback_to_prefix(R.k, R.v, R.a, R.b, self._S, self._S2, self.kv_len, R.n_keep, stream=st)
            self._S, self._S2 = self._S2, self._S
        self._kv_hi = lb
        return R

    def prefill(self, prompt, chunk: int = 8192):
        """Runs a prompt (int32 [B][P], one length for every request) through the layer, every
        row kept: the step before decoding.  The prompt goes in chunks of ``chunk`` tokens in
        order; per chunk the embedding, both projections and the split run over all of its
        rows at once (each row's bits are its bits at any M), GDN over the chunk's rows
        (xv_gdn_prefill) and attention over them (xv_attn_prefill, which appends the rows
        and advances the length), each row with the decode arithmetic; then the head, the
        greedy id and its logprob for the last prompt row.  ``chunk`` changes no bit of the
        result, which equals feeding the prompt one token at a time.  Returns (ids [B],
        logprobs [B]) of the first generated token (device tensors); the state, KV cache and
        lengths advance by P."""
        wl, st, dev = self.wl, self.stream, self.device
        prompt = np.ascontiguousarray(prompt, dtype=np.int32)
        B, P = prompt.shape
        if B != wl.B or P < 1 or chunk < 1:
            raise ValueError("prefill: bad prompt shape or chunk")
        self.settle()
        e = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=dev)
        f = lambda *sh: torch.empty(sh, dtype=torch.float32, device=dev)
        for c0 in range(0, P, chunk):
            cp = min(chunk, P - c0)
            M = B * cp
            ids = torch.from_numpy(np.ascontiguousarray(prompt[:, c0:c0 + cp]).reshape(-1)).to(dev)
            x, y1, y2 = e(M, wl.K), e(M, wl.N1), e(M, wl.N2)
            q, k, v = e(B, cp, wl.Hk, wl.dk), e(B, cp, wl.Hk, wl.dk), e(B, cp, wl.Hv, wl.dv)
            a, b = f(B, cp, wl.Hv), f(B, cp, wl.Hv)
            qa, kn, vn = e(B, cp, wl.Hq, wl.d), e(B, cp, wl.Hkv, wl.d), e(B, cp, wl.Hkv, wl.d)
            og, oa = e(B, cp, wl.Hv, wl.dv), e(B, cp, wl.Hq, wl.d)
            xv.xv_embed_rows(self.E, ids, x, stream=st)
            xv.xv_gemm_small_m_pair(x, self.W1, y1, None, x, self.W2, y2, None, stream=st)
            xv.xv_split_projections(y1, y2, q, k, v, a, b, qa, kn, vn, stream=st)
            xv.xv_gdn_prefill(q, k, v, a, b, self._S, self._S2, og, None, stream=st)
            self._S, self._S2 = self._S2, self._S
            xv.xv_attn_prefill(qa, kn, vn, self.Kc, self.Vc, self.kv_len, oa, None, self.scale, advance=True,
                               stream=st)
            self._kv_hi = min(self._kv_hi + cp, self.Lmax)
        # the head and the greedy id of each request's last prompt row (rows gathered by the
        # library's row-copy kernel)
        last = torch.from_numpy((np.arange(B, dtype=np.int32) * cp + cp - 1).astype(np.int32)).to(dev)
        xg, xa = e(B, wl.Hv * wl.dv), e(B, wl.Hq * wl.d)
        xv.xv_embed_rows(og.view(M, wl.Hv * wl.dv), last, xg, stream=st)
        xv.xv_embed_rows(oa.view(M, wl.Hq * wl.d), last, xa, stream=st)
        lg, la = e(B, wl.NH), e(B, wl.NH)
        lg32, la32 = f(B, wl.NH), f(B, wl.NH)
        out = torch.empty((B, 1), dtype=torch.int32, device=dev)
        nk = torch.empty((B,), dtype=torch.int32, device=dev)
        lp = f(B, 1)
        toks = torch.from_numpy(np.ascontiguousarray(prompt[:, P - 1:])).to(dev)
        xv.xv_head_greedy_accept(xg, self.Wh_g, lg, lg32, xa, self.Wh_a, la, la32, toks, out, nk,
                                 self._hg_ws(B, 1), logprob=lp, stream=st)
        return out[:, 0], lp[:, 0]

    def snapshot(self):
        """Copies of the decoding state (GDN state, KV cache, lengths)."""
        return (self.S.clone(), self.Kc.clone(), self.Vc.clone(), self.kv_len.clone())

    def restore(self, snap):
        S, Kc, Vc, kv = snap
        self._pending = None
        self._S.copy_(S); self.Kc.copy_(Kc); self.Vc.copy_(Vc); self.kv_len.copy_(kv)
        self._kv_hi = int(kv.max()) if kv.numel() else 0

    def generate(self, root: np.ndarray, n_tokens: int,
                 drafts: Optional[Callable[[int, int, int], np.ndarray]] = None, k: int = 0,
                 record: Optional[list] = None, logits: Optional[list] = None):
        """Greedy decoding of n_tokens per request from root (int32 [B]); drafts(b, pos, k)
        proposes k ids after request b's pos-th emitted token.  Reads each step's results
        back to the host.  Returns (ids int32 [B][n], logprobs fp32 [B][n], per-step n_keep);
        record, when given, receives each step's input tokens (int32 [B][k+1]); logits, when
        given, receives one list per request of the fp32 logits row of every emitted token."""
        B = self.wl.B
        out_ids = [[] for _ in range(B)]
        out_lp = [[] for _ in range(B)]
        keeps = []
        if logits is not None:
            logits.extend([] for _ in range(B))
        cur = np.asarray(root, np.int32).copy()
        while min(len(o) for o in out_ids) < n_tokens:
            tok = np.empty((B, k + 1), np.int32)
            tok[:, 0] = cur
            for bb in range(B):
                if k:
                    tok[bb, 1:] = drafts(bb, len(out_ids[bb]), k)
            if record is not None:
                record.append(tok.copy())
            R = self.rows(k + 1, self._slot)
            R.tokens.copy_(torch.from_numpy(tok))
            self.step(R.tokens)
            ids = R.ids.cpu().numpy()
            lp = R.lp.cpu().numpy()
            nk = R.n_keep.cpu().numpy()
            keeps.append(nk.copy())
            if logits is not None:
                z = (R.lg32 + R.la32).view(B, k + 1, -1).cpu().numpy()   # the fp32 sum the greedy kernel forms
            for bb in range(B):
                n = int(nk[bb])
                if logits is not None:
                    logits[bb].extend(z[bb, i].copy() for i in range(n))
                out_ids[bb].extend(int(i) for i in ids[bb, :n])
                out_lp[bb].extend(float(x) for x in lp[bb, :n])
                cur[bb] = ids[bb, n - 1]
        ids = np.array([o[:n_tokens] for o in out_ids], np.int32)
        lps = np.array([o[:n_tokens] for o in out_lp], np.float32)
        return ids, lps, keeps
