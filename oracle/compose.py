"""Composed greedy decoding on the synthetic hybrid layer, fp64 (oracle).

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests and the
smoke check call it; the product library never does.

What it follows.  The post (first paragraph, and the paragraph on the two
verify changes) reports that greedy decoding with speculative verification
produced the same token ids and the same logprobs as decoding without it.
This module runs both loops on one synthetic layer, built only from the
oracle's pinned primitives (``gemm``, ``gdn``, ``attn``, ``greedy``,
``logprob``) plus the plain steps below, so the claim can be checked on the
oracle itself and the GPU loop can be compared with it.

The synthetic layer (a reading: the pages describe the model only by name and
launch flags).  Per input token id:
  x     = E[id]                                     (bf16 row of the embedding table)
  y1    = bf16(x W1^T)   columns: GDN q (Hk*dk) | GDN k (Hk*dk) | GDN v (Hv*dv)
  y2    = bf16(x W2^T)   columns: attention q (Hq*d) | k (Hkv*d) | v (Hkv*d) |
                                  decay logit (Hv) | beta logit (Hv) | unused
  q, k  = bf16(u / sqrt(sum(u^2) + 1e-6)) per head (L2 normalisation)
  a     = fp32(1 / (1 + exp(alpha)))   (= exp(-softplus(alpha)))
  b     = fp32(1 / (1 + exp(-beta)))   (sigmoid)
  GDN verify on (q, k, v, a, b), state stored in fp32 after every token;
  attention rows on (q_attn, k_new, v_new) over the KV cache;
  logits = bf16(o_gdn) Wh_gdn^T + bf16(o_attn) Wh_attn^T;
  greedy ids, accepted drafts, logprob of each id.
A step consumes tokens[b] = [root, draft_1 .. draft_k], keeps n = 1 + accepted
rows (their GDN state, KV rows and length), and emits ids[b][0 .. n-1]; the
last emitted id is the next step's root.  Decoding without speculation is the
same step with k = 0.

Rounding to bf16 here is of the exact fp64 value (nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import attn, gdn, gemm, greedy, logprob

L2_EPS = 1e-6


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of fp64 values, as uint16 bit patterns (finite, normal range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)  # 8 significant bits; rint rounds half to even
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_value(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Shapes:
    Hk: int
    Hv: int
    dk: int
    dv: int
    Hq: int
    Hkv: int
    d: int


def split(y1: np.ndarray, y2: np.ndarray, s: Shapes):
    """Per-head operands of one layer from the projection rows (bf16 bits [M][N1], [M][N2]).

    Returns q, k (fp64, normalised, before bf16 rounding) [M][Hk][dk]; v bits [M][Hv][dv];
    a, b (fp64) [M][Hv]; q_attn bits [M][Hq][d]; k_new, v_new bits [M][Hkv][d].
    """
    M = y1.shape[0]
    nq = s.Hk * s.dk
    out = {}
    for name, off in (("q", 0), ("k", nq)):
        u = bf16_value(y1[:, off:off + nq]).reshape(M, s.Hk, s.dk)
        out[name] = u / np.sqrt(np.sum(u * u, axis=-1, keepdims=True) + L2_EPS)
    out["v"] = np.ascontiguousarray(y1[:, 2 * nq:2 * nq + s.Hv * s.dv]).reshape(M, s.Hv, s.dv)
    o = 0
    out["q_attn"] = np.ascontiguousarray(y2[:, o:o + s.Hq * s.d]).reshape(M, s.Hq, s.d); o += s.Hq * s.d
    out["k_new"] = np.ascontiguousarray(y2[:, o:o + s.Hkv * s.d]).reshape(M, s.Hkv, s.d); o += s.Hkv * s.d
    out["v_new"] = np.ascontiguousarray(y2[:, o:o + s.Hkv * s.d]).reshape(M, s.Hkv, s.d); o += s.Hkv * s.d
    alpha = bf16_value(y2[:, o:o + s.Hv]); o += s.Hv
    beta = bf16_value(y2[:, o:o + s.Hv])
    out["a"] = 1.0 / (1.0 + np.exp(alpha))
    out["b"] = 1.0 / (1.0 + np.exp(-beta))
    return out


@dataclass
class Model:
    E: np.ndarray        # bf16 [V][K]
    W1: np.ndarray       # bf16 [N1][K]
    W2: np.ndarray       # bf16 [N2][K]
    Wh_gdn: np.ndarray   # bf16 [V][Hv*dv]
    Wh_attn: np.ndarray  # bf16 [V][Hq*d]
    s: Shapes

    @property
    def scale(self) -> float:
        return 1.0 / np.sqrt(self.s.d)


@dataclass
class State:
    S: np.ndarray        # fp32 [B][Hv][dk][dv]
    kc: np.ndarray       # bf16 [B][Hkv][Lmax][d]
    vc: np.ndarray
    kv_len: np.ndarray   # int32 [B]

    def copy(self) -> "State":
        return State(self.S.copy(), self.kc.copy(), self.vc.copy(), self.kv_len.copy())


def step(m: Model, st: State, tokens: np.ndarray, keep_all: bool = False):
    """One verify step over tokens int32 [B][T]; updates ``st`` in place to the kept prefix
    (the greedy acceptance; every row with keep_all, as in ``prefill``).

    Returns (ids [B][T], logprobs fp64 [B][T], n_keep [B], logits fp64 [B][T][V]).
    """
    s = m.s
    B, T = tokens.shape
    M = B * T
    x = m.E[tokens.reshape(-1)]
    y1 = round_bf16(gemm(x, m.W1))
    y2 = round_bf16(gemm(x, m.W2))
    sp = split(y1, y2, s)
    q = round_bf16(sp["q"]).reshape(B, T, s.Hk, s.dk)
    k = round_bf16(sp["k"]).reshape(B, T, s.Hk, s.dk)
    v = sp["v"].reshape(B, T, s.Hv, s.dv)
    a = sp["a"].astype(np.float32).reshape(B, T, s.Hv)
    b = sp["b"].astype(np.float32).reshape(B, T, s.Hv)
    # GDN, one token at a time so that the state is stored in fp32 after every token
    o_gdn = np.empty((B, T, s.Hv, s.dv), np.float64)
    S_all = np.empty((T + 1,) + st.S.shape, np.float32)
    S_all[0] = st.S
    for t in range(T):
        sl = slice(t, t + 1)
        o_t, S_t, _ = gdn(q[:, sl].copy(), k[:, sl].copy(), v[:, sl].copy(), a[:, sl].copy(),
                          b[:, sl].copy(), S_all[t])
        o_gdn[:, t] = o_t[:, 0]
        S_all[t + 1] = S_t.astype(np.float32)
    qa = sp["q_attn"].reshape(B, T, s.Hq, s.d)
    kn = sp["k_new"].reshape(B, T, s.Hkv, s.d)
    vn = sp["v_new"].reshape(B, T, s.Hkv, s.d)
    o_attn = attn(qa, kn, vn, st.kc, st.vc, st.kv_len, m.scale)
    logits = (gemm(round_bf16(o_gdn).reshape(M, s.Hv * s.dv), m.Wh_gdn)
              + gemm(round_bf16(o_attn).reshape(M, s.Hq * s.d), m.Wh_attn)).reshape(B, T, -1)
    ids, n_keep = greedy(logits, np.ascontiguousarray(tokens, dtype=np.int32))
    if keep_all:
        n_keep = np.full((B,), T, np.int32)
    lp = logprob(logits, ids)
    for bb in range(B):
        n = int(n_keep[bb])
        L0 = int(st.kv_len[bb])
        st.S[bb] = S_all[n, bb]
        st.kc[bb, :, L0:L0 + n] = kn[bb, :n].transpose(1, 0, 2)
        st.vc[bb, :, L0:L0 + n] = vn[bb, :n].transpose(1, 0, 2)
        st.kv_len[bb] = L0 + n
    return ids, lp, n_keep, logits


def prefill(m: Model, st: State, prompt: np.ndarray):
    """The prompt (int32 [B][P]) through the layer with every row kept: the step before
    decoding, which leaves the GDN state, the KV cache and the length after the prompt
    (post, launch command: chunked prefill of 8192 tokens; the chunking is a schedule,
    not part of what is computed, so there is none here).  Returns (id [B], logprob [B],
    logits [B][V]) of the last prompt row: the first generated token.

    The rows are those of ``step`` with the acceptance replaced by "keep all P": one
    token at a time for the state (stored in fp32 after every token), attention rows
    over the cache, the head and the greedy id of each row.
    """
    P = prompt.shape[1]
    ids, lp, _, logits = step(m, st, np.ascontiguousarray(prompt, dtype=np.int32), keep_all=True)
    return ids[:, P - 1].copy(), lp[:, P - 1].copy(), logits[:, P - 1].copy()


def generate(m: Model, st: State, root: np.ndarray, n_tokens: int, drafts=None, k: int = 0):
    """Greedy decoding of n_tokens per request from ``root`` (int32 [B]).

    drafts(b, pos, k) -> k proposed ids for request b after its pos-th emitted token
    (k = 0: decoding without speculation).  Returns (ids int32 [B][n], logprobs [B][n],
    list of per-step n_keep, list of per-step min top-2 logit gaps [B]) and leaves ``st``
    at the end state.  Requests that reach n_tokens keep stepping with the others; only
    their first n_tokens emitted ids are returned.
    """
    B = root.shape[0]
    out_ids = [[] for _ in range(B)]
    out_lp = [[] for _ in range(B)]
    keeps, gaps = [], []
    cur = root.astype(np.int32).copy()
    while min(len(o) for o in out_ids) < n_tokens:
        tokens = np.empty((B, k + 1), np.int32)
        tokens[:, 0] = cur
        for bb in range(B):
            if k:
                tokens[bb, 1:] = drafts(bb, len(out_ids[bb]), k)
        ids, lp, n_keep, logits = step(m, st, tokens)
        srt = np.sort(logits, axis=-1)
        gaps.append((srt[..., -1] - srt[..., -2]).min(axis=-1))
        keeps.append(n_keep.copy())
        for bb in range(B):
            n = int(n_keep[bb])
            out_ids[bb].extend(int(i) for i in ids[bb, :n])
            out_lp[bb].extend(float(x) for x in lp[bb, :n])
            cur[bb] = ids[bb, n - 1]
    ids = np.array([o[:n_tokens] for o in out_ids], np.int32)
    lps = np.array([o[:n_tokens] for o in out_lp], np.float64)
    return ids, lps, keeps, gaps
