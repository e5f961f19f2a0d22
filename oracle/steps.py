"""The oracle's own composition of one workload step, per sequence.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): used by the full-size parity
tests and by the CPU-baseline leg of the benchmark.  It chains the fp64
functions of ``oracle.csa`` in the order of the DeepSeek-V4 method page
(section 3.3): the entries that complete are compressed and stored, the
indexer scores every visible entry, the top-k is taken, and the query attends
over the selected entries, the window rows and the sink.

Stored rows are rounded to their storage format (bf16 entries and window rows,
or mixed rows -- e4m3 codes under a row scale for the non-rotated dims, bf16 for
the rotated ones; e4m3 indexer keys with a per-row scale) because the caches
hold those bytes.
Inputs are fp64 arrays of the exact stored input values; the raw rows of the
entry cache are fetched on demand through a callable, so only the rows a
query touches are ever decoded.

Pins (tests/test_oracle_pins.py): each composition equals the plain
whole-sequence chain (compress every entry from all tokens, store, score,
select, attend) on small instances, with the cache's newest row planted stale
so that reading it fails; source mutations of the block offset, the replaced
row, the entry position and the window are shown to fail those pins.
"""
from __future__ import annotations

from typing import Callable

import numpy as np

from . import csa as O
from .codecs import e4m3_to_f64, f64_to_bf16_value, mx_fp4_to_f64


def _store(x: np.ndarray, dtype: str, rope_dim: int = 0) -> np.ndarray:
    """The value a cache row holds in storage format ``dtype`` ("mixed": the
    KV-entry format of the method page, section 3.3 -- see quantize_rows_mixed)."""
    if dtype == "mixed":
        return O.quantize_rows_mixed(x, rope_dim)[0]
    return f64_to_bf16_value(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def entry_rows(raw_rows: np.ndarray, s: np.ndarray, *, m: int, rope_dim: int, rope_base: float,
               eps: float, dtype: str, gamma=None) -> np.ndarray:
    """Cache rows built from pre-norm rows: RMSNorm (weight gamma, None = 1), RoPE at
    position m*s, storage rounding."""
    E = O.rope(O.rmsnorm(raw_rows, gamma, eps), m * np.asarray(s), rope_dim, rope_base)
    return _store(E, dtype, rope_dim)


def window_rows(raw_rows: np.ndarray, toks: np.ndarray, *, rope_dim: int, rope_base: float,
                eps: float, dtype: str, gamma=None) -> np.ndarray:
    W = O.rope(O.rmsnorm(raw_rows, gamma, eps), np.asarray(toks), rope_dim, rope_base)
    return _store(W, dtype, rope_dim)


def csa_decode_sequence(p: dict, kv_raw_rows: Callable[[np.ndarray], np.ndarray],
                        attend_idx=None) -> dict:
    """One CSA decode step of one sequence.

    ``attend_idx`` (optional, k indices with -1 padding) replaces the oracle's
    own top-k as the set the query attends over; the scores and the oracle's
    selection are still returned.  A selection that another implementation
    made from its own fp32 scores may differ at near-ties of the k-th score,
    and its attention output is still defined exactly.

    p holds: i, m, N, k, n_win, d_I, rope_dim, rope_base, eps, scale, dtype (storage of the
    entries and window rows: "bf16", "f32" or "mixed"), k_dtype;
    KI (N x d_I fp64, fp8 keys already times their scale; for MXFP4 keys
    instead KI_codes (N x d_I E2M1 codes) and KI_scales (N x d_I / 32 E8M0
    codes), scored on the FP4 query-key path), win_raw (n_win x d,
    tokens i-n_win+1..i), Ca/Za/Cb/Zb (2m x d, tokens m(N-2)..mN-1),
    ICa/IZa/ICb/IZb (2m x d_I), qI (H x d_I), w (H), q (n_h x d), sink (n_h); optionally
    gamma (d, the RMSNorm weight of the KV rows; default 1).
    kv_raw_rows(s) returns the pre-norm rows of entries s.
    """
    i, m, N, k, n_win = p["i"], p["m"], p["N"], p["k"], p["n_win"]
    r, base, eps = p["rope_dim"], p["rope_base"], p["eps"]
    T = m * N
    tok_base = m * (N - 2)
    # newest complete block: KV entry (norm + RoPE) and indexer key (no norm, stored format)
    gam = p.get("gamma")
    e_new = O.compress(p["Ca"], p["Za"], p["Cb"], p["Zb"], m=m, overlap=1, T=T, tok_base=tok_base,
                       s_begin=N - 1, s_end=N, gamma=gam, eps=eps, rope_dim=r, rope_base=base)[0]
    e_new = _store(e_new, p["dtype"], r)
    k_new = O.compress(p["ICa"], p["IZa"], p["ICb"], p["IZb"], m=m, overlap=1, T=T, tok_base=tok_base,
                       s_begin=N - 1, s_end=N, normalize=False)
    if p["k_dtype"] == "mxfp4":
        kc, ks = O.quantize_rows_mxfp4(k_new)
        KIc, KIs = p["KI_codes"].copy(), p["KI_scales"].copy()
        KIc[N - 1], KIs[N - 1] = kc[0], ks[0]
        k_new = mx_fp4_to_f64(kc, ks)
        I = O.index_score_mxfp4(p["qI"][None], p["w"][None], KIc, KIs, [i], m=m)
    else:
        if p["k_dtype"] == "e4m3":
            codes, sc = O.quantize_rows_e4m3(k_new)
            k_new = e4m3_to_f64(codes) * sc.astype(np.float64)[:, None]
        else:
            k_new = _store(k_new, p["k_dtype"])
        KI = p["KI"].copy()
        KI[N - 1] = k_new[0]
        I = O.index_score(p["qI"][None], p["w"][None], KI, [i], m=m)
    # top-k
    idx, vals = O.topk(I, [i], m=m, k=k)
    # rows the query reads
    use = idx[0] if attend_idx is None else np.asarray(attend_idx, dtype=np.int64)
    sel = use[use >= 0]
    rows = np.zeros((len(sel), p["q"].shape[-1]))
    old = sel[sel != N - 1]
    if len(old):
        rows[sel != N - 1] = entry_rows(kv_raw_rows(old), old, m=m, rope_dim=r, rope_base=base,
                                        eps=eps, dtype=p["dtype"], gamma=gam)
    rows[sel == N - 1] = e_new
    toks = np.arange(i - n_win + 1, i + 1)
    W = window_rows(p["win_raw"], toks, rope_dim=r, rope_base=base, eps=eps, dtype=p["dtype"], gamma=gam)
    out = O.attend_one(p["q"], np.concatenate([rows, W]), i=i, eps=eps, sink=p["sink"], rope_dim=r,
                       rope_base=base, scale=p["scale"])
    return {"I": I[0], "idx": idx[0], "vals": vals[0], "out": out, "k_new": k_new[0]}


def hca_decode_sequence(p: dict, kv_raw_rows: Callable[[np.ndarray], np.ndarray]) -> dict:
    """One HCA decode step of one sequence: recompress the just-completed block,
    then dense attention over every visible entry, the window and the sink.
    p holds: i, m, N, n_win, rope_dim, rope_base, eps, scale, dtype, C, Z (m x d),
    win_raw, q, sink; optionally gamma (d, the RMSNorm weight of the KV rows; default 1)."""
    i, m, N, n_win = p["i"], p["m"], p["N"], p["n_win"]
    r, base, eps = p["rope_dim"], p["rope_base"], p["eps"]
    n_vis = O.n_visible(i, m, N)
    s = np.arange(n_vis)
    gam = p.get("gamma")
    E = np.zeros((n_vis, p["q"].shape[-1]))
    E[: N - 1] = entry_rows(kv_raw_rows(s[: N - 1]), s[: N - 1], m=m, rope_dim=r, rope_base=base,
                            eps=eps, dtype=p["dtype"], gamma=gam)
    e_new = O.compress(p["C"], p["Z"], None, None, m=m, overlap=0, T=m * N, tok_base=m * (N - 1),
                       s_begin=N - 1, s_end=N, gamma=gam, eps=eps, rope_dim=r, rope_base=base)[0]
    E[N - 1] = _store(e_new, p["dtype"], r)
    toks = np.arange(i - n_win + 1, i + 1)
    W = window_rows(p["win_raw"], toks, rope_dim=r, rope_base=base, eps=eps, dtype=p["dtype"], gamma=gam)
    out = O.attend_one(p["q"], np.concatenate([E, W]), i=i, eps=eps, sink=p["sink"], rope_dim=r,
                       rope_base=base, scale=p["scale"])
    return {"out": out}


def csa_prefill_queries(p: dict, ts, kv_raw_rows: Callable[[np.ndarray], np.ndarray],
                        attend_idx=None) -> dict:
    """Chunked CSA prefill, evaluated for the chunk queries ``ts`` only.
    ``attend_idx`` (optional, [len(ts), k]) replaces the oracle's own
    selections as the sets the queries attend over (see csa_decode_sequence).

    The chunk holds queries at positions p0 .. p0 + Tq - 1.  Entries s0 = p0/m ..
    s1 = min(N, (p0 + Tq)/m) complete inside the chunk and are compressed from
    the chunk's candidates (KV entries with norm + RoPE, indexer keys without);
    earlier entries come from the cache.  Each query then scores every visible
    entry, takes its top-k and attends over those entries, its window and the sink.

    p holds: p0, Tq, m, N, k, n_win, rope_dim, rope_base, eps, scale, dtype, k_dtype;
    KI (N x d_I stored key values), tok_base, Ca/Za/Cb/Zb (rows of tokens
    tok_base ..), ICa/IZa/ICb/IZb, win_before (raw window rows of tokens
    p0 - n_win + 1 .. p0 - 1), chunk_raw (raw rows of tokens p0 .. p0 + Tq - 1),
    qI [len(ts), H, d_I], w [len(ts), H], q [len(ts), n_h, d], sink.
    kv_raw_rows(s) returns the pre-norm rows of cached entries s.
    """
    p0, Tq, m, N, k, n_win = p["p0"], p["Tq"], p["m"], p["N"], p["k"], p["n_win"]
    r, base, eps = p["rope_dim"], p["rope_base"], p["eps"]
    T = p0 + Tq
    s0, s1 = p0 // m, min(N, T // m)
    E_new = _store(O.compress(p["Ca"], p["Za"], p["Cb"], p["Zb"], m=m, overlap=1, T=T,
                              tok_base=p["tok_base"], s_begin=s0, s_end=s1, eps=eps,
                              rope_dim=r, rope_base=base), p["dtype"], r)
    K_new = _store(O.compress(p["ICa"], p["IZa"], p["ICb"], p["IZb"], m=m, overlap=1, T=T,
                              tok_base=p["tok_base"], s_begin=s0, s_end=s1, normalize=False),
                   p["k_dtype"])
    KI = p["KI"].copy()
    KI[s0:s1] = K_new
    tok_lo = p0 - (n_win - 1)
    W = window_rows(np.concatenate([p["win_before"], p["chunk_raw"]]), np.arange(tok_lo, T),
                    rope_dim=r, rope_base=base, eps=eps, dtype=p["dtype"])
    res = {"I": [], "idx": [], "out": []}
    for j, t in enumerate(ts):
        i = p0 + int(t)
        I = O.index_score(p["qI"][j][None], p["w"][j][None], KI, [i], m=m)
        idx, _ = O.topk(I, [i], m=m, k=k)
        use = idx[0] if attend_idx is None else np.asarray(attend_idx[j], dtype=np.int64)
        sel = use[use >= 0]
        rows = np.zeros((len(sel), p["q"].shape[-1]))
        old = sel < s0
        if old.any():
            rows[old] = entry_rows(kv_raw_rows(sel[old]), sel[old], m=m, rope_dim=r, rope_base=base,
                                   eps=eps, dtype=p["dtype"])
        rows[~old] = E_new[sel[~old] - s0]
        toks = np.arange(i - n_win + 1, i + 1)
        out = O.attend_one(p["q"][j], np.concatenate([rows, W[toks - tok_lo]]), i=i, eps=eps,
                           sink=p["sink"], rope_dim=r, rope_base=base, scale=p["scale"])
        res["I"].append(I[0])
        res["idx"].append(idx[0])
        res["out"].append(out)
    res = {key: np.stack(v) for key, v in res.items()}
    res.update(E_new=E_new, KI_new=K_new, s0=s0)
    return res
