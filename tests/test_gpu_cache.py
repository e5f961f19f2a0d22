"""Heterogeneous cache maintenance on the GPU (csa_cache_append, through the C ABI).

Three sequences start at different positions (per-sequence prefixes appended
through one-sequence views of the caches), then receive joint appends of mixed
sizes: 1 token (decode), 3, 130 (more than a tail ring), 64.  The caches --
CSA entries, indexer keys, HCA entries, the window ring and the tail ring --
must equal the oracle's compression of each whole sequence (method page
section 3.5: classical blocks of lcm(m, m') tokens plus a state cache), and a
second chunking of the same tokens must give the same bytes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import cache as Cc
from oracle import codecs as oc
from oracle import csa as O
from synth import Gen
from tests._util import TOL_BF16, row_rel_err, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("Ca", "Za", "Cb", "Zb", "ICa", "IZa", "ICb", "IZb", "Ch", "Zh", "Wraw")


@pytest.fixture(scope="module")
def csa():
    import long_context_attention_02_amd as lib
    return lib


def _caches(B, c, dI, N_csa, N_hca, W_cap, R, k_dtype):
    z = dict(device=DEV)
    st = dict(tail=torch.zeros((B, R, 6 * c + 4 * dI), dtype=torch.bfloat16, **z),
              E_csa=torch.full((B, N_csa, c), float("nan"), dtype=torch.bfloat16, **z),
              E_hca=torch.full((B, N_hca, c), float("nan"), dtype=torch.bfloat16, **z),
              W=torch.full((B, W_cap, c), float("nan"), dtype=torch.bfloat16, **z))
    if k_dtype == "mxfp4":
        st["K_idx"] = torch.zeros((B, N_csa, dI // 2), dtype=torch.uint8, **z)
        st["K_scale"] = torch.zeros((B, N_csa, dI // 32), dtype=torch.uint8, **z)
    else:
        st["K_idx"] = torch.full((B, N_csa, dI), float("nan"), dtype=torch.bfloat16, **z)
        st["K_scale"] = None
    return st


def _append(csa, st, tok, b_sl, t0, n, kw):
    """Append tokens t0[b] .. t0[b] + n - 1 of the sequences in b_sl."""
    new = {k: torch.stack([tok[k][b, t0[i]:t0[i] + n] for i, b in enumerate(range(b_sl.start, b_sl.stop))])
           .contiguous() for k in NAMES}
    T0 = torch.tensor(t0, dtype=torch.int32, device=DEV)
    csa.csa_cache_append(T0, new, st["tail"][b_sl], st["E_csa"][b_sl], st["K_idx"][b_sl], st["E_hca"][b_sl],
                         st["W"][b_sl], K_scale=None if st["K_scale"] is None else st["K_scale"][b_sl], **kw)


@pytest.mark.parametrize("k_dtype", ["bf16", "mxfp4"])
def test_cache_append_equals_full_recompression(csa, k_dtype):
    B, c, dI, m, m_hca, n_win, r = 3, 512, 128, 4, 128, 128, 64
    R = csa.cache_ring_slots(m, m_hca)
    prefix = [0, 5, 130]
    chunks = [1, 3, 130, 1, 64, 2]
    T_end = [p + sum(chunks) for p in prefix]
    N_csa, N_hca = max(T_end) // m + 2, max(T_end) // m_hca + 2
    g = Gen(880, DEV)
    Tmax = max(T_end)
    tok = {k: g.normal(i + 1, (B, Tmax, dI if k.startswith("I") else c), "bf16") for i, k in enumerate(NAMES)}
    gamma = (1.0 + 0.25 * g.normal(20, (c,), "f32", per_slot=False)).contiguous()
    kw = dict(m=m, m_hca=m_hca, gamma=gamma, eps=1e-6, rope_dim=r, rope_base=10000.0)

    def run(st, plan):
        t = [0] * B
        for b, p in enumerate(prefix):              # each sequence alone to its own start
            if p:
                _append(csa, st, tok, slice(b, b + 1), [0], p, kw)
                t[b] = p
        for n in plan:                              # then joint appends
            _append(csa, st, tok, slice(0, B), t, n, kw)
            t = [x + n for x in t]
        return t

    st = _caches(B, c, dI, N_csa, N_hca, n_win, R, k_dtype)
    assert run(st, chunks) == T_end
    torch.cuda.synchronize()
    gam = to_f64(gamma)
    for b in range(B):
        T = T_end[b]
        tb = {k: to_f64(tok[k][b]) for k in NAMES}
        # the oracle with gamma: scale its unit-gamma rows (RMSNorm is linear in gamma and
        # precedes RoPE, which mixes pairs: apply gamma before the rotation instead)
        n_csa, n_hca = T // m, T // m_hca
        E = O.compress(*(tb[k][:T] for k in ("Ca", "Za", "Cb", "Zb")), m=m, overlap=1, T=T, s_begin=0,
                       s_end=n_csa, gamma=gam, rope_dim=r)
        H = O.compress(tb["Ch"][:T], tb["Zh"][:T], None, None, m=m_hca, overlap=0, T=T, s_begin=0, s_end=n_hca,
                       gamma=gam, rope_dim=r)
        K = O.compress(*(tb[k][:T] for k in ("ICa", "IZa", "ICb", "IZb")), m=m, overlap=1, T=T, s_begin=0,
                       s_end=n_csa, normalize=False)
        assert row_rel_err(to_f64(st["E_csa"][b, :n_csa]), E) <= TOL_BF16, b
        assert torch.isnan(st["E_csa"][b, n_csa:].float()).all(), "entries of incomplete blocks stay unwritten"
        assert row_rel_err(to_f64(st["E_hca"][b, :n_hca]), H) <= TOL_BF16, b
        assert torch.isnan(st["E_hca"][b, n_hca:].float()).all()
        if k_dtype == "mxfp4":
            kc, ks = O.quantize_rows_mxfp4(K)
            got_s = st["K_scale"][b, :n_csa].cpu().numpy()
            assert np.mean(got_s == ks) > 0.99
            dec = oc.mx_fp4_to_f64(oc.unpack_fp4(st["K_idx"][b, :n_csa].cpu().numpy()), got_s)
            assert row_rel_err(dec, K) <= 0.25           # MXFP4 keeps about 2 significant bits
        else:
            assert row_rel_err(to_f64(st["K_idx"][b, :n_csa]), K) <= TOL_BF16, b
        toks = np.arange(T - n_win, T)
        Wr = O.rope(O.rmsnorm(tb["Wraw"][toks], gam, 1e-6), toks, r)
        assert row_rel_err(to_f64(st["W"][b][toks % n_win]), Wr) <= TOL_BF16, b
        # the tail ring holds the raw rows of the last R tokens, bit for bit
        tail = st["tail"][b].cpu()
        ref = Cc.cache_state({k: tb[k] for k in NAMES}, T, m=m, m_hca=m_hca, n_win=n_win, rope_dim=r,
                             rope_base=10000.0, eps=1e-6)["tail"]
        off = 0
        for k in NAMES[:-1]:
            w = dI if k.startswith("I") else c
            rows = ref[k]
            for u, t in enumerate(range(T - len(rows), T)):
                assert np.array_equal(to_f64(tail[t % R, off:off + w]), rows[u]), (b, k, t)
            off += w

    # another chunking of the same tokens: the same bytes everywhere
    st2 = _caches(B, c, dI, N_csa, N_hca, n_win, R, k_dtype)
    run(st2, [sum(chunks) - 7, 7])
    torch.cuda.synchronize()
    for key in ("E_csa", "E_hca", "W", "tail", "K_idx", "K_scale"):
        if st[key] is None:
            continue
        a, bb = st[key], st2[key]
        if a.dtype == torch.bfloat16:
            a, bb = torch.nan_to_num(a.float(), nan=7.0), torch.nan_to_num(bb.float(), nan=7.0)
        assert torch.equal(a, bb), key


def _sampled_entries_check(st, tok, b, t_lo, entries_csa, entries_hca, *, m, m_hca, gam, r, dI, n_win, T_end):
    """Entries (CSA with their keys, HCA) compressed by appends whose candidate tokens all lie at or
    after t_lo (rows tok[k][b][t - t_lo]), and the window rows of the last n_win tokens, against
    the oracle's compression of those tokens."""
    class _Rows:   # fp64 copies of just the rows asked for
        def __getitem__(self, k):
            return _Slicer(k)

    class _Slicer:
        def __init__(self, k):
            self.k = k

        def __getitem__(self, sl):
            return to_f64(tok[self.k][b][torch.as_tensor(np.arange(tok[self.k].shape[1])[sl], device=DEV)])

    rows = _Rows()
    for s in entries_csa:
        lo = m * (s - 1)
        assert lo >= t_lo
        sl = slice(lo - t_lo, m * (s + 1) - t_lo)
        E = O.compress(*(rows[k][sl] for k in ("Ca", "Za", "Cb", "Zb")), m=m, overlap=1, T=m * (s + 1),
                       tok_base=lo, s_begin=s, s_end=s + 1, gamma=gam, rope_dim=r)
        assert row_rel_err(to_f64(st["E_csa"][b, s:s + 1]), E) <= TOL_BF16, ("csa", s)
        K = O.compress(*(rows[k][sl] for k in ("ICa", "IZa", "ICb", "IZb")), m=m, overlap=1, T=m * (s + 1),
                       tok_base=lo, s_begin=s, s_end=s + 1, normalize=False)
        assert row_rel_err(to_f64(st["K_idx"][b, s:s + 1]), K) <= TOL_BF16, ("key", s)
    for h in entries_hca:
        lo = m_hca * h
        assert lo >= t_lo
        sl = slice(lo - t_lo, lo + m_hca - t_lo)
        H = O.compress(rows["Ch"][sl], rows["Zh"][sl], None, None, m=m_hca, overlap=0, T=lo + m_hca, tok_base=lo,
                       s_begin=h, s_end=h + 1, gamma=gam, rope_dim=r)
        assert row_rel_err(to_f64(st["E_hca"][b, h:h + 1]), H) <= TOL_BF16, ("hca", h)
    toks = np.arange(T_end - n_win, T_end)
    Wr = O.rope(O.rmsnorm(rows["Wraw"][toks - t_lo], gam, 1e-6), toks, r)
    assert row_rel_err(to_f64(st["W"][b][toks % n_win]), Wr) <= TOL_BF16


def test_cache_append_full_size_positions(csa):
    """At the Pro shapes (c = 512, d_I = 128, m = 4, m' = 128, window 128, RoPE on 64 dims):
    (1) two sequences reach position 2^20 - 1 with a 128-token append that fills the tail ring,
    then a one-token decode append completes CSA entry 262,143 and HCA entry 8,191 (RoPE at
    positions near 2^20, earlier tokens read back from the ring); (2) one sequence receives a
    16,384-token prefill chunk at position 114,688 (4,096 CSA entries, 128 HCA entries); sampled
    entries, every key sampled with them, and the window rows against the oracle."""
    c, dI, m, m_hca, n_win, r = 512, 128, 4, 128, 128, 64
    R = csa.cache_ring_slots(m, m_hca)
    g = Gen(890, DEV)
    gamma = (1.0 + 0.25 * g.normal(20, (c,), "f32", per_slot=False)).contiguous()
    gam = to_f64(gamma)
    kw = dict(m=m, m_hca=m_hca, gamma=gamma, eps=1e-6, rope_dim=r, rope_base=10000.0)
    # (1) decode at the 1M position
    B, T_last = 2, 1048575
    t_lo = T_last - 128
    tok = {k: g.normal(i + 1, (B, 129, dI if k.startswith("I") else c), "bf16") for i, k in enumerate(NAMES)}
    N_csa, N_hca = (T_last + 1) // m + 1, (T_last + 1) // m_hca + 1
    st = _caches(B, c, dI, N_csa, N_hca, n_win, R, "bf16")
    first = {k: tok[k][:, :128].contiguous() for k in NAMES}
    csa.csa_cache_append(torch.full((B,), t_lo, dtype=torch.int32, device=DEV), first, st["tail"], st["E_csa"],
                         st["K_idx"], st["E_hca"], st["W"], **kw)
    last = {k: tok[k][:, 128:].contiguous() for k in NAMES}
    csa.csa_cache_append(torch.full((B,), T_last, dtype=torch.int32, device=DEV), last, st["tail"], st["E_csa"],
                         st["K_idx"], st["E_hca"], st["W"], **kw)
    torch.cuda.synchronize()
    for b in range(B):
        _sampled_entries_check(st, tok, b, t_lo, [262142, 262143], [8191], m=m, m_hca=m_hca, gam=gam, r=r, dI=dI,
                               n_win=n_win, T_end=T_last + 1)
    del st, tok
    torch.cuda.empty_cache()
    # (2) a prefill chunk
    T0, n_new = 114688, 16384
    tok = {k: g.normal(40 + i, (1, n_new, dI if k.startswith("I") else c), "bf16") for i, k in enumerate(NAMES)}
    N_csa, N_hca = (T0 + n_new) // m + 1, (T0 + n_new) // m_hca + 1
    st = _caches(1, c, dI, N_csa, N_hca, n_win, R, "bf16")
    csa.csa_cache_append(torch.full((1,), T0, dtype=torch.int32, device=DEV), tok, st["tail"], st["E_csa"],
                         st["K_idx"], st["E_hca"], st["W"], **kw)
    torch.cuda.synchronize()
    s0, s1 = T0 // m + 1, (T0 + n_new) // m - 1        # entries whose sets lie inside the chunk
    csa_s = [s0, s0 + 1, (s0 + s1) // 2, s1 - 1, s1]
    h0, h1 = T0 // m_hca, (T0 + n_new) // m_hca - 1
    _sampled_entries_check(st, tok, 0, T0, csa_s, [h0, (h0 + h1) // 2, h1], m=m, m_hca=m_hca, gam=gam, r=r,
                           dI=dI, n_win=n_win, T_end=T0 + n_new)
    # the tail ring holds the raw rows of the last 128 tokens, bit for bit
    tail = st["tail"][0].cpu()
    off = 0
    for k in NAMES[:-1]:
        w = dI if k.startswith("I") else c
        for t in (T0 + n_new - 128, T0 + n_new - 1):
            assert torch.equal(tail[t % R, off:off + w].view(torch.uint8),
                               tok[k][0, t - T0].cpu().view(torch.uint8)), (k, t)
        off += w
