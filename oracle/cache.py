"""Heterogeneous cache maintenance, in fp64 (the oracle).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Source: "DeepSeek-V4: Towards Highly Efficient Million-Token Context
Intelligence", section 3.5: the inference cache is heterogeneous -- a classical
cache whose blocks each cover lcm(m, m') raw tokens (the compressed CSA
entries, their indexer keys and the HCA entries of those tokens) and a state
cache holding the sliding-window KV and the tokens of compression blocks that
are not yet complete.  Section 3.3 gives what each part holds (compressor,
window branch).

``cache_state`` is the plain definition: the caches after T tokens are the
compression of the whole sequence restricted to the entries whose blocks are
complete, the window rows of the last n_win tokens, and the raw rows of the
last lcm(m, m') tokens.  ``append_incremental`` maintains the same state token
by token from the previous state and a ring of lcm(m, m') raw-row slots only
(the reading of the state cache); a test pins the two against each other.
"""
from __future__ import annotations

import math

import numpy as np

from . import csa as O
from .codecs import f64_to_bf16_value

STREAMS_CSA = ("Ca", "Za", "Cb", "Zb")
STREAMS_IDX = ("ICa", "IZa", "ICb", "IZb")
STREAMS_HCA = ("Ch", "Zh")


def _store(x, dtype):
    return f64_to_bf16_value(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def ring_slots(m: int, m_hca: int) -> int:
    return m * m_hca // math.gcd(m, m_hca)


def cache_state(tok: dict, T: int, *, m: int, m_hca: int, n_win: int, rope_dim: int, rope_base: float,
                eps: float, dtype: str = "bf16") -> dict:
    """Caches after the first T tokens of a sequence.  tok[name] holds the raw
    per-token rows (>= T of them) of every stream: CSA candidates Ca, Za, Cb, Zb
    (c), indexer candidates ICa .. IZb (d_I), HCA candidates Ch, Zh (c) and the
    window rows Wraw (c).  Entry s of a compression is present once its block is
    complete: m (s + 1) <= T.  Keys are returned unrounded (their storage
    format is the caller's)."""
    n_csa, n_hca = T // m, T // m_hca
    c = tok["Ca"].shape[1]
    E = np.zeros((n_csa, c))
    K = np.zeros((n_csa, tok["ICa"].shape[1]))
    if n_csa:
        E = _store(O.compress(*(tok[k][:T] for k in STREAMS_CSA), m=m, overlap=1, T=T, s_begin=0,
                              s_end=n_csa, eps=eps, rope_dim=rope_dim, rope_base=rope_base), dtype)
        K = O.compress(*(tok[k][:T] for k in STREAMS_IDX), m=m, overlap=1, T=T, s_begin=0, s_end=n_csa,
                       normalize=False)
    H = np.zeros((n_hca, c))
    if n_hca:
        H = _store(O.compress(tok["Ch"][:T], tok["Zh"][:T], None, None, m=m_hca, overlap=0, T=T, s_begin=0,
                              s_end=n_hca, eps=eps, rope_dim=rope_dim, rope_base=rope_base), dtype)
    lo = max(0, T - n_win)
    Wr = _store(O.rope(O.rmsnorm(tok["Wraw"][lo:T], None, eps), np.arange(lo, T), rope_dim, rope_base), dtype)
    R = ring_slots(m, m_hca)
    tail = {k: tok[k][max(0, T - R):T] for k in STREAMS_CSA + STREAMS_IDX + STREAMS_HCA}
    return {"E_csa": E, "K_idx": K, "E_hca": H, "window": Wr, "window_tokens": np.arange(lo, T), "tail": tail}


def append_incremental(state: dict, ring: dict, new: dict, T0: int, *, m: int, m_hca: int, n_win: int,
                       rope_dim: int, rope_base: float, eps: float, dtype: str = "bf16") -> int:
    """Append the rows of new tokens T0 .. T0 + n - 1 to a state built so far
    (lists E_csa, K_idx, E_hca; dict window {token: row}) using only the ring of
    the last lcm(m, m') tokens' raw rows (ring[name][slot], slot = token mod the
    ring size) for the candidates of earlier tokens.  Returns T0 + n."""
    R = ring_slots(m, m_hca)
    n = new["Ca"].shape[0]
    for u in range(n):
        t = T0 + u
        for k in ring:
            ring[k][t % R] = new[k][u]

        def rows(names, lo, hi):
            # tokens lo .. hi - 1 of the given streams, read from the ring
            return [np.stack([ring[k][tt % R] for tt in range(lo, hi)]) for k in names]
        state["window"][t] = _store(O.rope(O.rmsnorm(new["Wraw"][u][None], None, eps), t, rope_dim,
                                           rope_base), dtype)[0]
        if (t + 1) % m == 0:                       # CSA entry s completes
            s = (t + 1) // m - 1
            lo = max(0, m * (s - 1))
            args = rows(STREAMS_CSA, lo, t + 1)
            E = O.compress(*args, m=m, overlap=1, T=t + 1, tok_base=lo, s_begin=s, s_end=s + 1, eps=eps,
                           rope_dim=rope_dim, rope_base=rope_base)
            state["E_csa"].append(_store(E[0], dtype))
            K = O.compress(*rows(STREAMS_IDX, lo, t + 1), m=m, overlap=1, T=t + 1, tok_base=lo, s_begin=s,
                           s_end=s + 1, normalize=False)
            state["K_idx"].append(K[0])
        if (t + 1) % m_hca == 0:                   # HCA entry h completes
            h = (t + 1) // m_hca - 1
            C, Z = rows(STREAMS_HCA, m_hca * h, t + 1)
            H = O.compress(C, Z, None, None, m=m_hca, overlap=0, T=t + 1, tok_base=m_hca * h, s_begin=h,
                           s_end=h + 1, eps=eps, rope_dim=rope_dim, rope_base=rope_base)
            state["E_hca"].append(_store(H[0], dtype))
        for old in [tt for tt in state["window"] if tt <= t - n_win]:
            del state["window"][old]
    return T0 + n
