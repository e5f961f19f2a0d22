"""Plain fp64 definition of the CSA/HCA attention core (the oracle).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``): slow, obviously correct,
numpy float64, one sequence at a time.  Inputs are fp64 arrays holding the
exact values of the stored bytes (decode them with ``oracle.codecs``).

Sources (cited by page title and section):

* [V4-abs §3.3]  "DeepSeek-V4: Towards Highly Efficient Million-Token Context
  Intelligence" (abstract / method summary page), section 3.3 "CSA and HCA
  hybrid attention": overlapping 1/m compressor with a row softmax over 2m
  elements; the lightning-indexer score formula; top-k; shared-KV MQA where an
  entry is both key and value; HCA = larger m', no overlap, dense attention;
  RMSNorm on query and KV entries; partial RoPE on the last 64 dims of query,
  entries and output, the output rotated again at position -i; a sliding-window
  branch of n_win uncompressed KV rows because a query cannot see its own block.
* [V4-abs §3.5]  same page, section 3.5: the state cache keeps the window KV
  and the tail tokens of the not-yet-full block.
* [V4-rep attn]  "DeepSeek V4 complete technical report" digest, section
  "hybrid attention: CSA + HCA": m = 4 / 128, top-k 512 / 1024, window 128,
  partial RoPE on the last 64 dims with -i on the output, learnable sink logits
  letting a head's total attention weight fall below 1.

Readings where the pages are silent are listed next to the code that takes
them (and collected in the design notes of the repository).
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import e4m3_code, f64_to_e4m3_value, mx_fp4_to_f64, mx_quantize_fp4

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# a1: compressor  [V4-abs §3.3], [V4-rep attn]
# ---------------------------------------------------------------------------
def candidate_tokens(s: int, m: int, overlap: int, T: int):
    """Tokens pooled into entry ``s``, as (set, token) pairs.

    Overlapping (CSA): set 'a' covers the entry's own block [m s, m(s+1)), set
    'b' the previous block [m(s-1), m s); both clipped to [0, T).  Every token
    then feeds exactly two entries and the rate is exactly 1/m (reading of the
    page's "two index ranges overlap").  Non-overlapping (HCA): only 'a'.
    """
    a = [("a", t) for t in range(m * s, min(m * (s + 1), T))]
    b = []
    if overlap:
        b = [("b", t) for t in range(max(m * (s - 1), 0), min(m * s, T))]
    return a + b


def num_entries(T: int, m: int) -> int:
    """Entries produced from T tokens: ceil(T/m) (a partial tail block still
    yields an entry; it stays invisible until its block is complete)."""
    return -(-T // m)


def pool_entries(Ca, Za, Cb, Zb, *, m: int, overlap: int, T: int, tok_base: int = 0,
                 s_begin: int = 0, s_end: int | None = None) -> np.ndarray:
    """Softmax-pooled entries before norm / RoPE, fp64 ``[s_end - s_begin, c]``.

    Row r of the candidate arrays holds token ``tok_base + r``.  For every
    entry and every channel j independently, the weights are a softmax over
    the candidate logits Z[., j] (max-subtracted) and the entry is the
    weighted sum of the candidates C[., j].  ``Z = None`` means all logits are
    0 (uniform weights).
    """
    Ca = np.asarray(Ca, dtype=np.float64)
    R, c = Ca.shape
    if s_end is None:
        s_end = num_entries(T, m)
    arrs = {"a": (Ca, Za), "b": (Cb, Zb)}
    out = np.zeros((s_end - s_begin, c))
    for s in range(s_begin, s_end):
        cands = candidate_tokens(s, m, overlap, T)
        if not cands:
            raise ValueError(f"entry {s} has no candidate token (T={T}, m={m})")
        C_rows, Z_rows = [], []
        for which, t in cands:
            r = t - tok_base
            if not 0 <= r < R:
                raise ValueError(f"token {t} of entry {s} is not among the given rows")
            C, Z = arrs[which]
            C_rows.append(np.asarray(C[r], dtype=np.float64))
            Z_rows.append(np.zeros(c) if Z is None else np.asarray(Z[r], dtype=np.float64))
        C = np.stack(C_rows)          # [n_cand, c]
        Z = np.stack(Z_rows)
        e = np.exp(Z - Z.max(axis=0, keepdims=True))
        alpha = e / e.sum(axis=0, keepdims=True)
        out[s - s_begin] = (alpha * C).sum(axis=0)
    return out


def rmsnorm(x, gamma=None, eps: float = 1e-6) -> np.ndarray:
    """x * gamma / sqrt(mean(x^2) + eps) over the last axis [V4-abs §3.3]."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y


def rope(x, pos, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """Rotate the last ``rope_dim`` dims of x at position ``pos``.

    Reading: adjacent pairs (2u, 2u+1) inside the last r dims turn by the
    angle pos * base^(-2u/r).  ``pos`` is a scalar or has x's leading shape.
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    d = x.shape[-1]
    r = rope_dim
    u = np.arange(r // 2, dtype=np.float64)
    theta = base ** (-2.0 * u / r)
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[..., None] * theta                  # [..., r/2]
    cos, sin = np.cos(ang), np.sin(ang)
    x0 = x[..., d - r + 0::2].copy()
    x1 = x[..., d - r + 1::2].copy()
    x[..., d - r + 0::2] = x0 * cos - x1 * sin
    x[..., d - r + 1::2] = x0 * sin + x1 * cos
    return x


def compress(Ca, Za, Cb, Zb, *, m: int, overlap: int, T: int, tok_base: int = 0,
             s_begin: int = 0, s_end: int | None = None, gamma=None, eps: float = 1e-6,
             rope_dim: int = 0, rope_base: float = 10000.0, pos_stride: int | None = None,
             pos_offset: int = 0, normalize: bool = True) -> np.ndarray:
    """Compressed entries: pool, then RMSNorm over c, then RoPE of the last
    ``rope_dim`` dims at position p_s = pos_stride*s + pos_offset.

    Reading: an entry's RoPE position is the first token of its own block
    (pos_stride = m, pos_offset = 0 by default).  ``normalize=False`` skips
    the norm (indexer keys are not normalised).
    """
    if s_end is None:
        s_end = num_entries(T, m)
    if pos_stride is None:
        pos_stride = m
    E = pool_entries(Ca, Za, Cb, Zb, m=m, overlap=overlap, T=T, tok_base=tok_base,
                     s_begin=s_begin, s_end=s_end)
    if normalize:
        E = rmsnorm(E, gamma, eps)
    pos = pos_stride * np.arange(s_begin, s_end) + pos_offset
    return rope(E, pos, rope_dim, rope_base)


def quantize_rows_e4m3(E) -> tuple[np.ndarray, np.ndarray]:
    """Store rows as e4m3fn codes with a per-row absmax scale.

    The code is an integer decided by floating point, so the decision is
    taken in fp32 like the stored format: scale = fp32(absmax) / 448 (1 for a
    zero row), code = RNE_sat(fp32(x) / scale).  Returns (codes uint8, scale
    float32).
    """
    x32 = np.asarray(E, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[..., None]).astype(np.float64)
    vals = f64_to_e4m3_value(y)
    return e4m3_code(vals), scale


# ---------------------------------------------------------------------------
# a2: lightning-indexer score  [V4-abs §3.3]
# ---------------------------------------------------------------------------
def n_visible(i: int, m: int, N_cap: int) -> int:
    """Entries visible to the query at absolute position i.

    Reading of "a query cannot see its own compressed block": entry s is
    visible iff its whole block is in the past, m(s+1) <= i+1.
    """
    return min(N_cap, (i + 1) // m)


def index_score(qI, w, K, q_pos, *, m: int, N_cap: int | None = None) -> np.ndarray:
    """I[t, s] = sum_h w[t,h] * ReLU(qI[t,h,:] . K[s,:]) for visible s, -inf
    elsewhere.

    qI: [Tq, H, dI], w: [Tq, H], K: [N_cap, dI] (fp8 keys already multiplied
    by their row scale), q_pos: [Tq] absolute positions.  Reading: no scale,
    no norm, K is shared by all indexer heads; masked entries are -inf, not 0,
    because a genuine score can be exactly 0.
    """
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if N_cap is None:
        N_cap = K.shape[0]
    Tq = qI.shape[0]
    out = np.full((Tq, N_cap), NEG_INF)
    for t in range(Tq):
        n = n_visible(int(q_pos[t]), m, N_cap)
        if n == 0:
            continue
        dots = qI[t] @ K[:n].T                     # [H, n]
        out[t, :n] = w[t] @ np.maximum(dots, 0.0)  # sum over heads
    return out


def quantize_rows_mixed(E, rope_dim: int):
    """Store KV rows in the mixed format [V4-abs §3.3: the KV entries keep their
    RoPE dims in BF16 and the rest in FP8]: the first c - rope_dim channels as
    e4m3fn codes with one per-row scale over them (absmax / 448, decided in fp32
    like ``quantize_rows_e4m3``), the last rope_dim channels rounded to bf16.
    Returns (stored values fp64 [..., c], codes uint8 [..., c - rope_dim], scale
    float32 [...])."""
    from .codecs import e4m3_to_f64, f64_to_bf16_value
    E = np.asarray(E, dtype=np.float64)
    nope = E.shape[-1] - rope_dim
    codes, sc = quantize_rows_e4m3(E[..., :nope])
    vals = np.concatenate([e4m3_to_f64(codes) * sc.astype(np.float64)[..., None],
                           f64_to_bf16_value(E[..., nope:])], axis=-1)
    return vals, codes, sc


def quantize_rows_mxfp4(E) -> tuple[np.ndarray, np.ndarray]:
    """Store rows in MXFP4 (OCP MX: E2M1 elements, one E8M0 scale per 32
    channels).  The decisions are taken on the fp32 value, the precision the
    pooled keys are computed in.  Returns (element codes uint8, scale codes
    uint8 [..., c / 32])."""
    x32 = np.asarray(E, dtype=np.float64).astype(np.float32).astype(np.float64)
    return mx_quantize_fp4(x32)


def index_score_mxfp4(qI, w, K_codes, K_scales, q_pos, *, m: int) -> np.ndarray:
    """The indexer score with the QK path in FP4 [V4-abs §3.6: the indexer's
    query-key path runs in FP4; §3.3: the score formula].

    Reading: both operands of every q . K product are MXFP4 -- the keys as
    stored (codes and block scales) and the query quantised from its stored
    (bf16) value by the OCP MX conversion, per head, blocks of 32 dims; the
    head weights stay fp32.  The score is then the plain formula on those
    values, I[t, s] = sum_h w[t,h] ReLU(q~[t,h] . K~[s]), exact in fp64.
    """
    qI = np.asarray(qI, dtype=np.float64)
    qc, qs = mx_quantize_fp4(qI)
    return index_score(mx_fp4_to_f64(qc, qs), w, mx_fp4_to_f64(K_codes, K_scales), q_pos, m=m)


# ---------------------------------------------------------------------------
# a3: top-k  [V4-abs §3.3], [V4-rep attn]
# ---------------------------------------------------------------------------
def topk(I, q_pos, *, m: int, k: int, N_cap: int | None = None):
    """Per row, the min(k, n_vis) visible indices with the largest score.

    Order: score descending, ties to the lower index; -0.0 equals +0.0.
    Missing slots are -1.  Returns (idx int64 [Tq, k], vals fp64 [Tq, k]).
    """
    I = np.asarray(I, dtype=np.float64)
    Tq = I.shape[0]
    if N_cap is None:
        N_cap = I.shape[1]
    idx = np.full((Tq, k), -1, dtype=np.int64)
    vals = np.full((Tq, k), NEG_INF)
    for t in range(Tq):
        n = n_visible(int(q_pos[t]), m, N_cap)
        row = I[t, :n]
        order = np.lexsort((np.arange(n), -row))   # primary: -score, then index
        sel = order[:min(k, n)]
        idx[t, :len(sel)] = sel
        vals[t, :len(sel)] = row[sel]
    return idx, vals


# ---------------------------------------------------------------------------
# a4 / a5: shared-KV MQA with window and sink  [V4-abs §3.3], [V4-rep attn]
# ---------------------------------------------------------------------------
def window_tokens(i: int, n_win: int):
    """Reading: the window is [i - n_win + 1, i], the query's own token
    included (its KV row is written before attention)."""
    return list(range(max(0, i - n_win + 1), i + 1))


def attend_one(q, KV, *, i: int, gamma_q=None, eps: float = 1e-6, sink=None,
               rope_dim: int = 0, rope_base: float = 10000.0, scale: float) -> np.ndarray:
    """Attention of one query (all heads) over its key set KV [n, d].

    q_hat = RoPE_i(RMSNorm(q_h)); l_j = scale * q_hat . kv_j; one softmax over
    the keys plus the sink: p_j = e^{l_j} / (e^{sigma_h} + sum_j e^{l_j});
    o = sum_j p_j kv_j (every row is both key and value); then the output's
    last r dims are rotated at position -i.  Reading: the sink has a zero
    value vector; with no key and no sink the output is 0.
    """
    q = np.asarray(q, dtype=np.float64)                 # [n_h, d]
    KV = np.asarray(KV, dtype=np.float64).reshape(-1, q.shape[-1])
    n_h, d = q.shape
    qh = rope(rmsnorm(q, gamma_q, eps), i, rope_dim, rope_base)
    out = np.zeros((n_h, d))
    for h in range(n_h):
        logits = scale * (KV @ qh[h])                   # [n]
        sig = None if sink is None else float(sink[h])
        if sig is not None and sig == -math.inf:
            sig = None
        terms = list(logits) + ([] if sig is None else [sig])
        if not terms:
            continue
        M = max(terms)
        e = np.exp(logits - M)
        Z = e.sum() + (0.0 if sig is None else math.exp(sig - M))
        out[h] = (e / Z) @ KV
    return rope(out, -i, rope_dim, rope_base)


def sparse_mqa(q, E, idx, W, *, q_pos, n_win: int, W_cap: int | None = None, gamma_q=None,
               eps: float = 1e-6, sink=None, rope_dim: int = 0, rope_base: float = 10000.0,
               scale: float) -> np.ndarray:
    """CSA core attention: key set = selected entries (idx != -1) plus the
    window rows, token tau read from W[tau mod W_cap].  Reading: one joint
    softmax over both groups and the sink."""
    q = np.asarray(q, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    Tq = q.shape[0]
    if W_cap is None and W is not None:
        W_cap = W.shape[0]
    out = np.zeros_like(q)
    for t in range(Tq):
        i = int(q_pos[t])
        rows = [E[s] for s in np.asarray(idx[t]) if 0 <= s < E.shape[0]]
        if n_win > 0:
            rows += [W[tau % W_cap] for tau in window_tokens(i, n_win)]
        KV = np.stack(rows) if rows else np.zeros((0, q.shape[-1]))
        out[t] = attend_one(q[t], KV, i=i, gamma_q=gamma_q, eps=eps, sink=sink,
                            rope_dim=rope_dim, rope_base=rope_base, scale=scale)
    return out


def dense_mqa(q, E, W, *, q_pos, m: int, n_win: int, W_cap: int | None = None, gamma_q=None,
              eps: float = 1e-6, sink=None, rope_dim: int = 0, rope_base: float = 10000.0,
              scale: float) -> np.ndarray:
    """HCA core attention: every visible entry s < n_vis(i) plus the window
    rows, one softmax with the sink [V4-abs §3.3: HCA keeps dense attention,
    otherwise as CSA]."""
    E = np.asarray(E, dtype=np.float64)
    Tq = np.asarray(q).shape[0]
    N_cap = E.shape[0]
    idx = [list(range(n_visible(int(q_pos[t]), m, N_cap))) for t in range(Tq)]
    width = max([len(r) for r in idx] + [1])
    idx_arr = np.full((Tq, width), -1, dtype=np.int64)
    for t, r in enumerate(idx):
        idx_arr[t, :len(r)] = r
    return sparse_mqa(q, E, idx_arr, W, q_pos=q_pos, n_win=n_win, W_cap=W_cap,
                      gamma_q=gamma_q, eps=eps, sink=sink, rope_dim=rope_dim,
                      rope_base=rope_base, scale=scale)
