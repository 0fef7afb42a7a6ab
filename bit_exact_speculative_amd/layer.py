"""One hybrid layer's speculative verify step on the GPU, built from libxv calls.

A :class:`Layer` holds the device buffers of one workload (weights, GDN state,
KV cache, the verify rows) and runs, on one stream:

  verify()  the hot path of one speculative step:
              x W1^T, x W2^T                     (xv_gemm_small_m_pair, M = B*T)
              GDN verify S_in -> S_out, o_gdn    (xv_gdn_verify)
              attention rows + KV append         (xv_attn_verify_rows)
              synthetic head logits, greedy ids, logprobs, accepted rows
                                                 (xv_head_greedy_accept on o_gdn and o_attn)
              rollback to the accepted prefix    (xv_rollback_to_prefix)
  lazy_step()  the same step with the rollback folded into the next step's GDN
              launch (the kept rows are replayed there; the greedy kernel adds
              them to the KV length), and GDN and attention in one call
              (xv_gdn_attn_verify); settle() runs the last pending rollback.
  decode_sequence()  the same layer advanced one token at a time (T = 1, M = B)
              over the same rows, which verify must reproduce bit for bit.

Torch provides device memory and the stream; every arithmetic step is a libxv
kernel.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import xv
from .inputs import Inputs, PREFIX_TOKENS


def dev_bf16(a: np.ndarray, device) -> torch.Tensor:
    """Upload bf16 bit patterns (uint16) as a torch.bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


class Layer:
    def __init__(self, inp: Inputs, device="cuda", state_in: Optional[np.ndarray] = None,
                 with_gemm: bool = True, with_head: bool = True, stream=None):
        wl = inp.wl
        self.wl = wl
        self.inp = inp
        self.device = device
        self.stream = stream
        B, T = wl.B, wl.T
        self.B, self.T = B, T
        g = inp.gdn
        self.q = dev_bf16(g["q"], device)
        self.k = dev_bf16(g["k"], device)
        self.v = dev_bf16(g["v"], device)
        self.a = dev(g["a"], device)
        self.b = dev(g["b"], device)
        self.S_in = torch.empty((B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=device)
        if state_in is not None:
            self.S_in.copy_(torch.from_numpy(np.ascontiguousarray(state_in, dtype=np.float32)))
        else:
            self.prefix_state_on_device()
        self.S_out = torch.empty_like(self.S_in)
        self.o_gdn = torch.empty((B, T, wl.Hv, wl.dv), dtype=torch.bfloat16, device=device)
        self.o_gdn32 = torch.empty((B, T, wl.Hv, wl.dv), dtype=torch.float32, device=device)
        # attention
        self.Lmax = inp.Lmax
        self.qa = dev_bf16(inp.q_attn, device)
        self.kn = dev_bf16(inp.k_new, device)
        self.vn = dev_bf16(inp.v_new, device)
        self.Kc0 = dev_bf16(inp.k_cache, device)            # pre-verify cache (kept)
        self.Vc0 = dev_bf16(inp.v_cache, device)
        self.Kc = self.Kc0.clone()
        self.Vc = self.Vc0.clone()
        self.L0 = dev(inp.L0.astype(np.int32), device)
        self.kv_len = self.L0.clone()
        # host upper bound on max(kv_len): each step adds at most T rows; the attention
        # launch is sized for kv_hi + T positions instead of the capacity (the same bits)
        self.L0_max = int(inp.L0.max()) if B else 0
        self.kv_hi = self.L0_max
        self.use_len_bound = True
        self.o_attn = torch.empty((B, T, wl.Hq, wl.d), dtype=torch.bfloat16, device=device)
        self.o_attn32 = torch.empty((B, T, wl.Hq, wl.d), dtype=torch.float32, device=device)
        self.ws = xv.xv_attn_workspace(B, T, wl.Hq, wl.d, self.Lmax, device)
        self.scale = 1.0 / float(wl.d) ** 0.5
        self.has_gemm = with_gemm and inp.x is not None
        if self.has_gemm:
            M = wl.M
            self.x = dev_bf16(inp.x, device)
            self.W1 = dev_bf16(inp.W1, device)
            self.W2 = dev_bf16(inp.W2, device)
            self.y1 = torch.empty((M, wl.N1), dtype=torch.bfloat16, device=device)
            self.y1_32 = torch.empty((M, wl.N1), dtype=torch.float32, device=device)
            self.y2 = torch.empty((M, wl.N2), dtype=torch.bfloat16, device=device)
            self.y2_32 = torch.empty((M, wl.N2), dtype=torch.float32, device=device)
        self.has_head = with_head and inp.Wh_gdn is not None
        if self.has_head:
            M = wl.M
            self.Wh_g = dev_bf16(inp.Wh_gdn, device)
            self.Wh_a = dev_bf16(inp.Wh_attn, device)
            self.lg = torch.empty((M, wl.NH), dtype=torch.bfloat16, device=device)
            self.lg32 = torch.empty((M, wl.NH), dtype=torch.float32, device=device)
            self.la = torch.empty((M, wl.NH), dtype=torch.bfloat16, device=device)
            self.la32 = torch.empty((M, wl.NH), dtype=torch.float32, device=device)
            self.draft = dev(inp.draft, device)
            self.ids = torch.empty((B, T), dtype=torch.int32, device=device)
            self.lp = torch.empty((B, T), dtype=torch.float32, device=device)
            self.hg_ws = torch.zeros((xv.xv_head_greedy_workspace_bytes(B, T, wl.NH),), dtype=torch.uint8,
                                     device=device)
        self.n_keep = torch.full((B,), T, dtype=torch.int32, device=device)
        self.pending = False         # lazy mode: S_in -> S_out ran, its rollback has not
        self.S_kept = None           # lazy mode: the two further state buffers
        self.S_next = None
        self.kv_scratch = None       # lazy mode: the pending rollback's KV count goes here
        self.proj_fp32 = True        # also write the fp32 projection outputs
        self.out_fp32 = True         # also write the fp32 GDN / attention outputs

    # ------------------------------------------------------------------
    def prefix_state_on_device(self):
        """S_in <- the GDN state after the 32-token prefix from a zero state (GPU path)."""
        wl, d = self.wl, self.device
        p = self.inp.prefix
        B = wl.B
        S = torch.zeros((B, wl.Hv, wl.dk, wl.dv), dtype=torch.float32, device=d)
        S2 = torch.empty_like(S)
        n = PREFIX_TOKENS
        t0 = 0
        while t0 < n:
            tt = min(16, n - t0)
            sl = slice(t0, t0 + tt)
            o = torch.empty((B, tt, wl.Hv, wl.dv), dtype=torch.bfloat16, device=d)
            xv.xv_gdn_verify(dev_bf16(p["q"][:, sl], d), dev_bf16(p["k"][:, sl], d),
                             dev_bf16(p["v"][:, sl], d), dev(p["a"][:, sl], d), dev(p["b"][:, sl], d),
                             S, S2, o, None, stream=self.stream)
            S, S2 = S2, S
            t0 += tt
        self.S_in.copy_(S)

    def reset(self):
        """Back to the pre-verify cache and lengths (the state buffers are not touched)."""
        self.Kc.copy_(self.Kc0)
        self.Vc.copy_(self.Vc0)
        self.kv_len.copy_(self.L0)
        self.kv_hi = self.L0_max

    def len_bound(self) -> int:
        """The attention calls' len_bound: max(kv_len) + T at most (0: size for the capacity)."""
        return min(self.kv_hi + self.T, self.Lmax) if self.use_len_bound else 0

    def _grew(self):
        """A call added up to T rows to kv_len."""
        self.kv_hi = min(self.kv_hi + self.T, self.Lmax)

    # ------------------------------------------------------------------
    def gemm1(self):
        xv.xv_gemm_small_m(self.x, self.W1, self.y1, self.y1_32 if self.proj_fp32 else None,
                           stream=self.stream)

    def gemm2(self, events=None):
        """events: optional (start, stop) torch.cuda.Event pair timed by the launch itself."""
        if events is None:
            xv.xv_gemm_small_m(self.x, self.W2, self.y2, self.y2_32 if self.proj_fp32 else None,
                               stream=self.stream)
        else:
            xv.xv_gemm_small_m_timed(self.x, self.W2, self.y2, self.y2_32 if self.proj_fp32 else None,
                                     events[0], events[1], stream=self.stream)

    def gemms(self, events=None):
        """Both projections in one launch (the bits of gemm1 and gemm2); events: optional
        (start, stop) torch.cuda.Event pair timed by the launch itself."""
        st = events if events is not None else (None, None)
        xv.xv_gemm_small_m_pair(self.x, self.W1, self.y1, self.y1_32 if self.proj_fp32 else None,
                                self.x, self.W2, self.y2, self.y2_32 if self.proj_fp32 else None,
                                st[0], st[1], stream=self.stream)

    def gdn(self):
        xv.xv_gdn_verify(self.q, self.k, self.v, self.a, self.b, self.S_in, self.S_out,
                         self.o_gdn, self.o_gdn32 if self.out_fp32 else None, stream=self.stream)

    def attn(self):
        xv.xv_attn_verify_rows(self.qa, self.kn, self.vn, self.Kc, self.Vc, self.kv_len,
                               self.o_attn, self.o_attn32 if self.out_fp32 else None, self.ws,
                               self.scale, len_bound=self.len_bound(), stream=self.stream)

    def head_gemms(self):
        """Both halves of the synthetic head in one launch."""
        wl, M = self.wl, self.wl.M
        xv.xv_gemm_small_m_pair(self.o_gdn.view(M, wl.Hv * wl.dv), self.Wh_g, self.lg, self.lg32,
                                self.o_attn.view(M, wl.Hq * wl.d), self.Wh_a, self.la, self.la32,
                                stream=self.stream)

    def greedy(self, count_kv: bool = False):
        """count_kv: the kernel also adds the kept rows to kv_len (lazy mode)."""
        wl = self.wl
        xv.xv_greedy_accept(self.lg32.view(self.B, self.T, wl.NH), self.la32.view(self.B, self.T, wl.NH),
                            self.draft, self.ids, self.n_keep, self.lp, stream=self.stream,
                            kv_len=self.kv_len if count_kv else None)
        if count_kv:
            self._grew()

    def head_greedy(self, count_kv: bool = False):
        """head_gemms() and greedy(count_kv) in one xv_head_greedy_accept call (the same bits)."""
        wl, M = self.wl, self.wl.M
        xv.xv_head_greedy_accept(self.o_gdn.view(M, wl.Hv * wl.dv), self.Wh_g, self.lg, self.lg32,
                                 self.o_attn.view(M, wl.Hq * wl.d), self.Wh_a, self.la, self.la32,
                                 self.draft, self.ids, self.n_keep, self.hg_ws, logprob=self.lp,
                                 kv_len=self.kv_len if count_kv else None, stream=self.stream)
        if count_kv:
            self._grew()

    def gdn_lazy(self):
        """GDN of a lazy step: the first one is xv_gdn_verify; later ones replay the previous
        step's kept rows (the same row buffers, n_keep from its greedy) from its start state,
        then run this step's rows (xv_gdn_verify_after).  S_in / S_out are the pending step's
        start state and S_T afterwards."""
        if self.S_kept is None:
            self.S_kept, self.S_next = torch.empty_like(self.S_in), torch.empty_like(self.S_in)
            self.kv_scratch = torch.zeros_like(self.kv_len)
        if not self.pending:
            self.gdn()
            self.pending = True
            return
        xv.xv_gdn_verify_after(self.q, self.k, self.v, self.a, self.b, self.k, self.v, self.a, self.b,
                               self.n_keep, self.S_in, self.S_out, self.S_kept, self.S_next,
                               self.o_gdn, self.o_gdn32 if self.out_fp32 else None, stream=self.stream)
        self.S_in, self.S_out, self.S_kept, self.S_next = self.S_kept, self.S_next, self.S_in, self.S_out

    def gdn_attn_lazy(self):
        """gdn_lazy() and attn() in one xv_gdn_attn_verify call (the same bits)."""
        if self.S_kept is None:
            self.S_kept, self.S_next = torch.empty_like(self.S_in), torch.empty_like(self.S_in)
            self.kv_scratch = torch.zeros_like(self.kv_len)
        if self.pending:
            out = self.S_next
            prev = (self.k, self.v, self.a, self.b, self.n_keep, self.S_out, self.S_kept)
        else:
            out, prev = self.S_out, None
        xv.xv_gdn_attn_verify(self.q, self.k, self.v, self.a, self.b, self.S_in, out, self.o_gdn,
                              self.qa, self.kn, self.vn, self.Kc, self.Vc, self.kv_len, self.o_attn, self.ws,
                              self.scale, o32=self.o_gdn32 if self.out_fp32 else None,
                              o_attn32=self.o_attn32 if self.out_fp32 else None, prev=prev,
                              len_bound=self.len_bound(), stream=self.stream)
        if self.pending:
            self.S_in, self.S_out, self.S_kept, self.S_next = self.S_kept, self.S_next, self.S_in, self.S_out
        self.pending = True

    def lazy_step(self, events=None):
        """One speculative step with the rollback deferred to the next step's GDN launch."""
        if not self.has_head:
            raise ValueError("a lazy step needs the head: its acceptance counts the kept rows")
        if self.has_gemm:
            self.gemms(events)
        self.gdn_attn_lazy()
        self.head_greedy(count_kv=True)

    def settle(self):
        """Lazy mode: the pending rollback (state only; the greedy kernel counted the KV
        rows), then S_in is the kept state as after verify + rollback + advance."""
        if not self.pending:
            return
        xv.xv_rollback_to_prefix(self.k, self.v, self.a, self.b, self.S_in, self.S_out, self.kv_scratch,
                                 self.n_keep, stream=self.stream)
        self.advance()
        self.pending = False

    def head(self):
        self.head_greedy()

    def rollback(self, n_keep: Optional[torch.Tensor] = None):
        xv.xv_rollback_to_prefix(self.k, self.v, self.a, self.b, self.S_in, self.S_out, self.kv_len,
                                 self.n_keep if n_keep is None else n_keep, stream=self.stream)
        self._grew()

    def verify(self, n_keep: Optional[torch.Tensor] = None, rollback: bool = True):
        """One speculative step; n_keep overrides the greedy acceptance when given."""
        if self.has_gemm:
            self.gemms()
        self.gdn()
        self.attn()
        if self.has_head:
            self.head()
        if rollback:
            self.rollback(n_keep)

    def advance(self):
        """After verify + rollback: the kept state becomes the next step's input state."""
        self.S_in, self.S_out = self.S_out, self.S_in

    def clone(self) -> "Layer":
        """A second layer with the same contents in separate device buffers."""
        other = Layer.__new__(Layer)
        for key, val in self.__dict__.items():
            other.__dict__[key] = val.clone() if isinstance(val, torch.Tensor) else val
        return other

    # ------------------------------------------------------------------
    def decode_sequence(self, n_tokens: Optional[int] = None):
        """Advance the layer one token at a time over rows 0..n-1 of every request.

        Uses fresh copies of the pre-verify cache, lengths and state; returns a
        dict of per-token outputs stacked on a token axis (torch tensors).
        """
        wl, d, st = self.wl, self.device, self.stream
        B, T = self.B, self.T
        n = T if n_tokens is None else n_tokens
        Kc = self.Kc0.clone(); Vc = self.Vc0.clone(); kv = self.L0.clone()
        S = self.S_in.clone(); S2 = torch.empty_like(S)
        one = torch.ones((B,), dtype=torch.int32, device=d)
        ws = xv.xv_attn_workspace(B, 1, wl.Hq, wl.d, self.Lmax, d)
        out = {k: [] for k in ("o_gdn", "o_gdn32", "S", "o_attn", "o_attn32", "kv_len",
                               "y1", "y1_32", "y2", "y2_32", "lg32", "la32", "ids", "lp")}
        for t in range(n):
            sl = slice(t, t + 1)
            q, k, v = self.q[:, sl].contiguous(), self.k[:, sl].contiguous(), self.v[:, sl].contiguous()
            a, b = self.a[:, sl].contiguous(), self.b[:, sl].contiguous()
            og = torch.empty((B, 1, wl.Hv, wl.dv), dtype=torch.bfloat16, device=d)
            og32 = torch.empty((B, 1, wl.Hv, wl.dv), dtype=torch.float32, device=d)
            xv.xv_gdn_verify(q, k, v, a, b, S, S2, og, og32, stream=st)
            S, S2 = S2, S
            oa = torch.empty((B, 1, wl.Hq, wl.d), dtype=torch.bfloat16, device=d)
            oa32 = torch.empty((B, 1, wl.Hq, wl.d), dtype=torch.float32, device=d)
            xv.xv_attn_verify_rows(self.qa[:, sl].contiguous(), self.kn[:, sl].contiguous(),
                                   self.vn[:, sl].contiguous(), Kc, Vc, kv, oa, oa32, ws, self.scale,
                                   stream=st)
            # the decode step keeps its one row: S unchanged (n == T), kv_len += 1
            xv.xv_rollback_to_prefix(k, v, a, b, S2, S, kv, one, stream=st)
            out["o_gdn"].append(og[:, 0].clone()); out["o_gdn32"].append(og32[:, 0].clone())
            out["S"].append(S.clone())
            out["o_attn"].append(oa[:, 0].clone()); out["o_attn32"].append(oa32[:, 0].clone())
            out["kv_len"].append(kv.clone())
            if self.has_gemm:
                xt = self.x.view(B, T, wl.K)[:, t].contiguous()
                y1 = torch.empty((B, wl.N1), dtype=torch.bfloat16, device=d)
                y1_32 = torch.empty((B, wl.N1), dtype=torch.float32, device=d)
                y2 = torch.empty((B, wl.N2), dtype=torch.bfloat16, device=d)
                y2_32 = torch.empty((B, wl.N2), dtype=torch.float32, device=d)
                xv.xv_gemm_small_m(xt, self.W1, y1, y1_32, stream=st)
                xv.xv_gemm_small_m(xt, self.W2, y2, y2_32, stream=st)
                out["y1"].append(y1); out["y1_32"].append(y1_32)
                out["y2"].append(y2); out["y2_32"].append(y2_32)
            if self.has_head:
                lg = torch.empty((B, wl.NH), dtype=torch.bfloat16, device=d)
                lg32 = torch.empty((B, wl.NH), dtype=torch.float32, device=d)
                la = torch.empty((B, wl.NH), dtype=torch.bfloat16, device=d)
                la32 = torch.empty((B, wl.NH), dtype=torch.float32, device=d)
                xv.xv_gemm_small_m(og.view(B, wl.Hv * wl.dv), self.Wh_g, lg, lg32, stream=st)
                xv.xv_gemm_small_m(oa.view(B, wl.Hq * wl.d), self.Wh_a, la, la32, stream=st)
                ids = torch.empty((B, 1), dtype=torch.int32, device=d)
                nk = torch.empty((B,), dtype=torch.int32, device=d)
                lp = torch.empty((B, 1), dtype=torch.float32, device=d)
                dr = self.draft[:, sl].contiguous()
                xv.xv_greedy_accept(lg32.view(B, 1, wl.NH), la32.view(B, 1, wl.NH), dr, ids, nk, lp, stream=st)
                out["lg32"].append(lg32); out["la32"].append(la32); out["ids"].append(ids[:, 0].clone())
                out["lp"].append(lp[:, 0].clone())
        res = {}
        for kname, vals in out.items():
            if vals:
                res[kname] = torch.stack(vals, dim=1 if kname not in ("S", "kv_len") else 0)
        res["Kc"] = Kc
        res["Vc"] = Vc
        return res
