"""Planted mistakes in a copy of the oracle must fail the pins (CPU only).

Each mutant is a one-line edit of oracle/xo.c of the kind a port could make:
a dropped term, a flipped sign, a swapped operand or index, an off-by-one in the
visible range, a wrong head mapping, a tie broken the other way.  The copy is
compiled to a temporary library, swapped in for the oracle, and every pin in
test_oracle_pins.py is run; at least one must fail.  No mutant reads outside
its buffers.
"""
import os

import pytest

import oracle
import tests.test_oracle_pins as pins

MUTANTS = [
    ("gemm_wrong_k", "s += xo_bf16(xr[k]) * xo_bf16(wr[k]);",
     "s += xo_bf16(xr[k]) * xo_bf16(wr[K - 1 - k]);"),
    ("gemm_transposed_out", "long m = e / N, n = e % N;", "long m = e % M, n = e / M;"),
    ("gdn_sign", "double p = S[(size_t)j * dk + i] - bt * Sk[j] * kt[i];",
     "double p = S[(size_t)j * dk + i] + bt * Sk[j] * kt[i];"),
    ("gdn_drop_write", "S[(size_t)j * dk + i] = at * p + bt * vj * kt[i];",
     "S[(size_t)j * dk + i] = at * p;"),
    ("gdn_drop_decay", "S[(size_t)j * dk + i] = at * p + bt * vj * kt[i];",
     "S[(size_t)j * dk + i] = p + bt * vj * kt[i];"),
    ("gdn_decay_on_write", "S[(size_t)j * dk + i] = at * p + bt * vj * kt[i];",
     "S[(size_t)j * dk + i] = at * (p + bt * vj * kt[i]);"),
    ("gdn_query_is_key", "for (int i = 0; i < dk; ++i) s += S[(size_t)j * dk + i] * qt[i];",
     "for (int i = 0; i < dk; ++i) s += S[(size_t)j * dk + i] * kt[i];"),
    ("gdn_head_map", "int g = h / (Hv / Hk);", "int g = h % Hk;"),
    ("gdn_state_transposed", "S[(size_t)j * dk + i] = (double)S0[((size_t)h * dk + i) * dv + j];",
     "S[(size_t)j * dk + i] = (double)S0[((size_t)h * dv + j) * dk + i];"),
    ("gdn_no_beta_in_erase", "double p = S[(size_t)j * dk + i] - bt * Sk[j] * kt[i];",
     "double p = S[(size_t)j * dk + i] - Sk[j] * kt[i];"),
    ("attn_sees_one_row", "long len = L0 + r + 1;", "long len = L0 + 1;"),
    ("attn_no_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("attn_kv_head_map", "int g = h / (Hq / Hkv);", "int g = h % Hkv;"),
    ("attn_cache_boundary", "const uint16_t* kr = (j < L0)", "const uint16_t* kr = (j <= L0 && j < Lmax)"),
    ("attn_no_normalise", "for (int e = 0; e < d; ++e) out[e] /= den;", "for (int e = 0; e < d; ++e) out[e] /= 1.0;"),
    ("greedy_tie_high", "if (row[n] > row[best]) best = n;", "if (row[n] >= row[best]) best = n;"),
    ("greedy_keep_off_by_one", "n_keep[bb] = acc + 1;", "n_keep[bb] = acc;"),
    ("greedy_compare_same_row",
     "while (acc + 1 < T && draft[(size_t)bb * T + acc + 1] == ids[(size_t)bb * T + acc]) ++acc;",
     "while (acc + 1 < T && draft[(size_t)bb * T + acc] == ids[(size_t)bb * T + acc]) ++acc;"),
    ("rollback_no_length", "for (int bb = 0; bb < B; ++bb) kv_out[bb] = kv_len[bb] + n_keep[bb];",
     "for (int bb = 0; bb < B; ++bb) kv_out[bb] = kv_len[bb];"),
    ("rollback_all_rows", "if (n > T) n = T;", "n = T;"),
    ("logprob_no_shift_in_sum", "for (int n = 0; n < N; ++n) s += exp(row[n] - m);",
     "for (int n = 0; n < N; ++n) s += exp(row[n]);"),
    ("logprob_first_index", "lp[r] = (row[ids[r]] - m) - log(s);", "lp[r] = (row[0] - m) - log(s);"),
    ("logprob_sign", "lp[r] = (row[ids[r]] - m) - log(s);", "lp[r] = (row[ids[r]] - m) + log(s);"),
]


def _all_pins():
    calls = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argname, values = params[0].args
            for v in values:
                calls.append((name, fn, {argname: v}))
        else:
            calls.append((name, fn, {}))
    return calls


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation site not unique: " + name
    mut_c = tmp_path / "xo_mut.c"
    mut_c.write_text(src.replace(old, new))
    so = oracle.compile_c(str(mut_c), str(tmp_path / "libxo_mut.so"))
    monkeypatch.setattr(oracle, "_lib", oracle._bind(so))
    caught = []
    for pname, fn, kw in _all_pins():
        try:
            fn(**kw)
        except Exception:        # assertion or arithmetic failure both count
            caught.append(pname)
    assert caught, "planted mistake %s passed every pin" % name
