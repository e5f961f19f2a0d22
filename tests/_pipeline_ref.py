"""Oracle inputs for the device-resident workload steps.

Decodes the exact stored bytes of a pipeline's inputs (never its outputs) into
the fp64 dictionaries that ``oracle.steps`` takes, and checks a selection
against the oracle's scores.
"""
from __future__ import annotations

import numpy as np
import torch

from tests._util import TOL_F32, to_f64


def _raw_rows(raw_b: torch.Tensor):
    def rows(s):
        return to_f64(raw_b[torch.as_tensor(np.asarray(s), device=raw_b.device)])
    return rows


def csa_decode_params(run, b: int):
    """(p, kv_raw_rows) of sequence b of a CSADecode run, for oracle.steps.csa_decode_sequence."""
    wl = run.wl
    keys = {}
    if wl.k_dtype == "mxfp4":
        # the oracle quantises the raw fp32 keys itself (never the device's cache bytes)
        from oracle import csa as O
        keys["KI_codes"], keys["KI_scales"] = O.quantize_rows_mxfp4(to_f64(run.KI_raw[b]))
    else:
        KI = to_f64(run.KI[b])
        if run.KI_scale is not None:
            KI = KI * to_f64(run.KI_scale[b])[:, None]
        keys["KI"] = KI
    p = dict(i=run.i, m=wl.m, N=wl.N_cap, k=wl.k, n_win=wl.n_win, d_I=wl.d_I, rope_dim=wl.rope_dim,
             rope_base=wl.rope_base, eps=wl.eps, scale=wl.scale, dtype=wl.kv_dtype, k_dtype=wl.k_dtype,
             **keys, win_raw=to_f64(run.win_raw[b]),
             Ca=to_f64(run.Ca[b]), Za=to_f64(run.Za[b]), Cb=to_f64(run.Cb[b]), Zb=to_f64(run.Zb[b]),
             ICa=to_f64(run.ICa[b]), IZa=to_f64(run.IZa[b]), ICb=to_f64(run.ICb[b]),
             IZb=to_f64(run.IZb[b]), qI=to_f64(run.qI[b, 0]), w=to_f64(run.wI[b, 0]),
             q=to_f64(run.q[b, 0]), sink=to_f64(run.sink), gamma=to_f64(run.gamma_kv))
    return p, _raw_rows(run.kv_raw[b])


def hca_decode_params(run, b: int):
    """(p, kv_raw_rows) of sequence b of an HCADecode run, for oracle.steps.hca_decode_sequence."""
    wl = run.wl
    p = dict(i=run.i, m=wl.m, N=wl.N_cap, n_win=wl.n_win, rope_dim=wl.rope_dim,
             rope_base=wl.rope_base, eps=wl.eps, scale=wl.scale, dtype=wl.kv_dtype,
             C=to_f64(run.C[b]), Z=to_f64(run.Z[b]), win_raw=to_f64(run.win_raw[b]),
             q=to_f64(run.q[b, 0]), sink=to_f64(run.sink), gamma=to_f64(run.gamma_kv))
    return p, _raw_rows(run.kv_raw[b])


def csa_prefill_params(run, ts):
    """(p, kv_raw_rows) of the chunk queries ts of a CSAPrefill run (sequence 0),
    for oracle.steps.csa_prefill_queries."""
    wl = run.wl
    ts_t = torch.as_tensor(np.asarray(ts), device=run.q.device)
    p = dict(p0=wl.q_pos0, Tq=wl.Tq, m=wl.m, N=wl.N_cap, k=wl.k, n_win=wl.n_win,
             rope_dim=wl.rope_dim, rope_base=wl.rope_base, eps=wl.eps, scale=wl.scale,
             dtype=wl.kv_dtype, k_dtype=wl.k_dtype, KI=to_f64(run.KI_init[0]), tok_base=run.tok_base,
             Ca=to_f64(run.Ca[0]), Za=to_f64(run.Za[0]), Cb=to_f64(run.Cb[0]), Zb=to_f64(run.Zb[0]),
             ICa=to_f64(run.ICa[0]), IZa=to_f64(run.IZa[0]), ICb=to_f64(run.ICb[0]),
             IZb=to_f64(run.IZb[0]), win_before=to_f64(run.win_raw[0]),
             chunk_raw=to_f64(run.chunk_raw[0]), qI=to_f64(run.qI[0, ts_t]), w=to_f64(run.wI[0, ts_t]),
             q=to_f64(run.q[0, ts_t]), sink=to_f64(run.sink))
    return p, _raw_rows(run.kv_raw[0])


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits); 0 maps to the smallest normal's."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))


def score_slack(qI: np.ndarray, w: np.ndarray, K_stored: np.ndarray) -> np.ndarray:
    """Bound on |I| change when each element of bf16-stored keys moves by one ulp.

    Keys that a step compresses and stores in bf16 are rounded from fp32 on the
    device and from fp64 in the oracle, so a value close to a rounding midpoint
    can land one ulp apart.  For query row qI [H, d_I] with weights w [H]:
    slack[s] = sum_h |w_h| * sum_d |qI[h, d]| * ulp(K[s, d])."""
    return (np.abs(w)[:, None] * np.abs(qI)).sum(axis=0) @ bf16_ulp(K_stored).T


def new_key_slack(qI: np.ndarray, w: np.ndarray, k_new: np.ndarray, k_dtype: str) -> float:
    """score_slack of the one key a decode step compresses: one storage ulp per
    element (bf16, or e4m3 times the row scale: k_new holds code * scale, and
    the scale's own fp32 rounding is far below an e4m3 ulp)."""
    if k_dtype == "f32":
        return 0.0
    if k_dtype == "bf16":
        return float(score_slack(qI, w, k_new[None])[0])
    if k_dtype == "mxfp4":
        # an E2M1 spacing per element at its block scale (doubled: near a power of two
        # the block scale itself may differ by one step), against the MXFP4 query
        from oracle import codecs as oc
        qc, qs = oc.mx_quantize_fp4(qI)
        qq = oc.mx_fp4_to_f64(qc, qs)
        kc, ks = oc.mx_quantize_fp4(k_new.astype(np.float32).astype(np.float64))
        X = np.repeat(oc.e8m0_to_f64(ks), 32, axis=-1)
        y = np.abs(k_new) / X
        ulp = 2.0 * np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0)) * X
        return float((np.abs(w)[:, None] * np.abs(qq)).sum(axis=0) @ ulp)
    from tests._util import e4m3_ulp
    sc = np.max(np.abs(k_new)) / 448.0
    ulp = e4m3_ulp(k_new / sc) * sc if sc > 0 else np.zeros_like(k_new)
    return float((np.abs(w)[:, None] * np.abs(qI)).sum(axis=0) @ ulp)


def check_selection(got_idx: np.ndarray, ref_idx: np.ndarray, ref_I: np.ndarray,
                    slack: np.ndarray | None = None) -> int:
    """A device selection against the oracle's, where each side scored the entries itself.

    Entries whose oracle scores lie within delta = 4 * TOL_F32 * max|I| of the
    k-th oracle score may trade places (rounding of the fp32 scores decides
    them); every other entry must be selected on both sides, in an order that
    the oracle scores confirm up to delta.  ``slack`` (per entry, absolute)
    widens the band for entries whose stored keys were rounded on each side
    separately (``score_slack``).  Returns the number of such swaps."""
    got = got_idx[got_idx >= 0]
    ref = ref_idx[ref_idx >= 0]
    assert len(got) == len(ref), ("selection size", len(got), len(ref))
    assert np.all(got_idx[len(got):] == -1), "padding"
    assert len(set(got.tolist())) == len(got), "duplicate index"
    fin = np.isfinite(ref_I)
    delta = 4 * TOL_F32 * float(np.max(np.abs(ref_I[fin]))) if fin.any() else 0.0
    assert np.all(fin[got]), "selected an invisible entry"
    sl = np.zeros(len(ref_I)) if slack is None else np.asarray(slack, dtype=np.float64)
    diff = set(got.tolist()) ^ set(ref.tolist())
    if len(ref):
        kth = ref_I[ref[-1]]
        for s in diff:
            band = delta + sl[s] + sl[ref[-1]]
            assert abs(ref_I[s] - kth) <= band, ("swap outside the rounding band", s, ref_I[s], kth)
        sc = ref_I[got]
        band = delta + sl[got][1:] + sl[got][:-1]
        assert np.all(sc[1:] <= sc[:-1] + band), "device order is not score-descending"
    return len(diff) // 2
