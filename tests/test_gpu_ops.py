"""GPU parity of each HIP entry point against the fp64 oracle, through the C ABI.

Inputs come from the seeded generators (``synth``); the very same bytes go to
the HIP path and, decoded exactly, to the oracle.  Sizes span several tiles of
every kernel path and end in ragged tails.  Tolerances: 1e-5 (fp32 outputs),
2e-2 (bf16 outputs), row-relative; top-k indices bit-exact.
"""
import math

import numpy as np
import pytest
import torch

from oracle import csa as O
from synth import Gen
from tests._util import TOL_BF16, TOL_F32, e4m3_ulp, row_rel_err, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def csa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_attention_02_amd as lib
    return lib


def _gamma(g, tid, c):
    # gamma around 1 so the norm's weight is exercised
    return (1.0 + 0.25 * g.normal(tid, (c,), "f32", per_slot=False)).contiguous()


# ---------------------------------------------------------------------------
# a1 compressor
# ---------------------------------------------------------------------------
COMPRESS_CASES = [
    # name, B, T, R, tok_base, c, m, overlap, s_begin, s_end, in, out, norm, rope, ring, z
    ("tiny_f32_kv", 1, 256, 256, 0, 64, 4, 1, 0, 64, "f32", "f32", True, 16, 0, True),
    ("tiny_f32_indexer_keys", 1, 256, 256, 0, 32, 4, 1, 0, 64, "f32", "f32", False, 0, 0, True),
    ("csa_bf16_ragged_tail", 3, 203, 203, 0, 512, 4, 1, 0, 51, "bf16", "bf16", True, 64, 0, True),
    ("csa_bf16_window_of_rows", 2, 1000, 44, 960 - 4, 128, 4, 1, 240, 250, "bf16", "f32", True, 32, 0, True),
    ("hca_bf16_tail_recompress", 4, 1048576, 128, 1048448, 512, 128, 0, 8191, 8192, "bf16", "bf16", True, 64, 0, True),
    ("hca_bf16_partial_block", 2, 300, 300, 0, 256, 128, 0, 0, 3, "bf16", "bf16", True, 64, 0, True),
    ("window_rows_m1_ring", 2, 300, 300, 0, 512, 1, 0, 172, 300, "bf16", "bf16", True, 64, 128, False),
    ("uniform_weights_no_Z", 1, 64, 64, 0, 96, 4, 1, 0, 16, "f32", "f32", False, 0, 0, False),
    # 256 or more (sequence, entry) pairs: the wave-per-entry kernel
    ("many_csa_bf16_entries", 2, 2050, 2050, 0, 512, 4, 1, 0, 513, "bf16", "bf16", True, 64, 0, True),
    ("many_csa_f32_entries_to_bf16", 1, 1203, 1203, 0, 64, 4, 1, 0, 301, "f32", "bf16", True, 16, 0, True),
    ("many_window_rows_ring", 2, 700, 700, 0, 512, 1, 0, 300, 700, "bf16", "bf16", True, 64, 512, False),
    ("many_entries_tail_rows", 1, 1400, 1032, 368, 128, 4, 1, 93, 350, "bf16", "f32", False, 0, 0, True),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=[c[0] for c in COMPRESS_CASES])
def test_compress_parity(csa, case):
    name, B, T, R, tok_base, c, m, ov, s0, s1, idt, odt, norm, rope, ring, use_z = case
    g = Gen(100 + COMPRESS_CASES.index(case), DEV)
    Ca = g.normal(1, (B, R, c), idt)
    Za = g.normal(2, (B, R, c), idt) if use_z else None
    Cb = g.normal(3, (B, R, c), idt) if ov else None
    Zb = g.normal(4, (B, R, c), idt) if (ov and use_z) else None
    gamma = _gamma(g, 5, c) if norm else None
    rows = ring if ring else s1
    E = torch.full((B, rows, c), float("nan"), dtype=TDT[odt], device=DEV)
    csa.csa_compress(Ca, Za, Cb, Zb, E, T=T, m=m, overlap=ov, s_begin=s0, s_end=s1, tok_base=tok_base,
                     gamma=gamma, eps=1e-6, rope_dim=rope, out_ring=ring)
    torch.cuda.synchronize()
    got = to_f64(E)
    gam = None if gamma is None else to_f64(gamma)
    tol = TOL_F32 if odt == "f32" else TOL_BF16
    for b in range(B):
        ref = O.compress(to_f64(Ca[b]), None if Za is None else to_f64(Za[b]),
                         None if Cb is None else to_f64(Cb[b]), None if Zb is None else to_f64(Zb[b]),
                         m=m, overlap=ov, T=T, tok_base=tok_base, s_begin=s0, s_end=s1, gamma=gam,
                         eps=1e-6, rope_dim=rope, normalize=norm)
        out_rows = [(s % ring) if ring else s for s in range(s0, s1)]
        # a ring keeps only the last `ring` entries
        keep = list(range(len(out_rows)))[-ring:] if ring else list(range(len(out_rows)))
        err = row_rel_err(got[b][[out_rows[r] for r in keep]], ref[keep])
        assert err <= tol, (name, b, err)
    if not ring:  # rows before s_begin are untouched
        assert torch.isnan(E[:, :s0]).all()


def test_compress_fp8_output(csa):
    """Indexer keys stored as e4m3fn with a per-row absmax scale: the code must be
    a correct RNE rounding of the oracle value (up to midpoint ties of the
    fp32-vs-fp64 pooled value)."""
    B, T, c, m = 3, 400, 128, 4
    g = Gen(150, DEV)
    Ca, Za, Cb, Zb = (g.normal(i, (B, T, c), "bf16") for i in (1, 2, 3, 4))
    n = O.num_entries(T, m)
    E = torch.zeros((B, n, c), dtype=torch.float8_e4m3fn, device=DEV)
    S = torch.zeros((B, n), dtype=torch.float32, device=DEV)
    csa.csa_compress(Ca, Za, Cb, Zb, E, T=T, m=m, overlap=1, s_begin=0, s_end=n, E_scale=S)
    torch.cuda.synchronize()
    codes = to_f64(E)
    scale = to_f64(S)
    mism = 0
    for b in range(B):
        ref = O.compress(*(to_f64(x[b]) for x in (Ca, Za, Cb, Zb)), m=m, overlap=1, T=T, normalize=False)
        rc, rs = O.quantize_rows_e4m3(ref)
        assert np.allclose(scale[b], rs, rtol=2e-6, atol=0)
        y = ref / scale[b][:, None]                      # oracle value in code units
        dec = codes[b]
        assert np.all(np.abs(dec - y) <= 0.5 * e4m3_ulp(y) * (1 + 1e-3) + 1e-6 * 448)
        mism += int(np.sum(to_f64(torch.from_numpy(rc).view(torch.float8_e4m3fn)) != dec))
    assert mism <= 0.001 * B * n * c


def test_compress_batch_matches_separate_calls(csa):
    """One launch of several jobs (a decode step's window row, KV entry and
    indexer key, plus an HCA block and an empty job) writes exactly the bytes
    of the separate calls, and those match the oracle."""
    g = Gen(160, DEV)
    B, c, cI, m, T = 3, 512, 128, 4, 4 * 37 + 2
    n = O.num_entries(T, m)
    Ca, Za, Cb, Zb = (g.normal(i, (B, T, c), "bf16") for i in (1, 2, 3, 4))
    ICa, IZa, ICb, IZb = (g.normal(i, (B, T, cI), "bf16") for i in (5, 6, 7, 8))
    Wr = g.normal(9, (B, T, c), "bf16")
    H = g.normal(10, (B, 256, c), "bf16")
    HZ = g.normal(11, (B, 256, c), "bf16")
    gamma = _gamma(g, 12, c)

    def outputs():
        return dict(E=torch.full((B, n, c), float("nan"), dtype=torch.bfloat16, device=DEV),
                    K=torch.zeros((B, n, cI), dtype=torch.float8_e4m3fn, device=DEV),
                    S=torch.zeros((B, n), dtype=torch.float32, device=DEV),
                    W=torch.full((B, 16, c), float("nan"), dtype=torch.bfloat16, device=DEV),
                    Hc=torch.full((B, 2, c), float("nan"), dtype=torch.bfloat16, device=DEV))

    def jobs(o):
        return [
            (Wr, None, None, None, o["W"], dict(T=T, m=1, overlap=0, s_begin=T - 16, s_end=T, gamma=gamma,
                                                 rope_dim=64, out_ring=16)),
            (Ca, Za, Cb, Zb, o["E"], dict(T=T, m=m, overlap=1, s_begin=0, s_end=n, gamma=gamma, rope_dim=64)),
            (ICa, IZa, ICb, IZb, o["K"], dict(T=T, m=m, overlap=1, s_begin=n - 5, s_end=n, E_scale=o["S"])),
            (H, HZ, None, None, o["Hc"], dict(T=256, m=128, overlap=0, s_begin=0, s_end=2, gamma=gamma,
                                              rope_dim=64)),
            (Ca, Za, Cb, Zb, o["E"], dict(T=T, m=m, overlap=1, s_begin=3, s_end=3)),   # empty
        ]

    sep, bat = outputs(), outputs()
    for C_a, Z_a, C_b, Z_b, E, kw in jobs(sep):
        csa.csa_compress(C_a, Z_a, C_b, Z_b, E, **kw)
    csa.csa_compress_batch(jobs(bat))
    torch.cuda.synchronize()
    for key in sep:
        a_, b_ = sep[key], bat[key]
        if a_.dtype == torch.float8_e4m3fn:
            a_, b_ = a_.view(torch.uint8), b_.view(torch.uint8)
        assert torch.equal(torch.nan_to_num(a_.float(), nan=7.0), torch.nan_to_num(b_.float(), nan=7.0)), key
    # and the batch against the oracle (the KV entries and the HCA block)
    gam = to_f64(gamma)
    for b in range(B):
        ref = O.compress(*(to_f64(x[b]) for x in (Ca, Za, Cb, Zb)), m=m, overlap=1, T=T, gamma=gam,
                         eps=1e-6, rope_dim=64)
        assert row_rel_err(to_f64(bat["E"][b]), ref) <= TOL_BF16
        refh = O.compress(to_f64(H[b]), to_f64(HZ[b]), None, None, m=128, overlap=0, T=256, gamma=gam,
                          eps=1e-6, rope_dim=64)
        assert row_rel_err(to_f64(bat["Hc"][b]), refh) <= TOL_BF16


# ---------------------------------------------------------------------------
# a2 indexer score
# ---------------------------------------------------------------------------
INDEX_CASES = [
    # name, B, Tq, H, dI, N, m, qdt, kdt, positions
    ("tiny_f32_prefill", 1, 256, 2, 32, 64, 4, "f32", "f32", "prefill0"),
    ("bf16_decode_h64_d128", 2, 1, 64, 128, 5000, 4, "bf16", "bf16", "all"),
    ("fp8_decode_h64_d128_masked", 3, 1, 64, 128, 7000, 4, "bf16", "e4m3", "partial"),
    ("bf16_decode_tq3_h32_d64", 2, 3, 32, 64, 3001, 4, "bf16", "bf16", "partial"),
    ("bf16_decode_h16_d32", 1, 2, 16, 32, 999, 1, "bf16", "bf16", "all"),
    ("bf16_prefill_h64_d128", 1, 45, 64, 128, 700, 4, "bf16", "bf16", "prefill"),
    ("fp8_prefill_h64_d128", 2, 20, 64, 128, 333, 4, "bf16", "e4m3", "prefill"),
    ("bf16_prefill_h32_d64", 1, 17, 32, 64, 260, 2, "bf16", "bf16", "prefill"),
    ("bf16_generic_h8_d48", 2, 5, 8, 48, 300, 4, "bf16", "bf16", "partial"),
    ("fp8_generic_h48_d128", 1, 3, 48, 128, 500, 4, "bf16", "e4m3", "all"),
]


def _positions(mode, B, Tq, N, m, g):
    if mode == "all":
        base = N * m
        p = [[base + t for t in range(Tq)] for _ in range(B)]
    elif mode == "partial":   # some entries invisible, different per row
        p = [[m * (N // 2 + 37 * b) + 3 * t + b for t in range(Tq)] for b in range(B)]
    elif mode == "prefill0":
        p = [[t for t in range(Tq)] for _ in range(B)]
    else:                     # a chunk ending near the cache's end; crosses many block boundaries
        p = [[m * N - Tq * 3 + 3 * t + b for t in range(Tq)] for b in range(B)]
    return torch.tensor(p, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("case", INDEX_CASES, ids=[c[0] for c in INDEX_CASES])
def test_index_score_parity(csa, case):
    name, B, Tq, H, dI, N, m, qdt, kdt, pmode = case
    g = Gen(200 + INDEX_CASES.index(case), DEV)
    qI = g.normal(1, (B, Tq, H, dI), qdt)
    w = g.uniform(2, (B, Tq, H))
    Ks = None
    if kdt == "e4m3":
        K, Ks = g.normal_e4m3(3, (B, N, dI))
    else:
        K = g.normal(3, (B, N, dI), kdt)
    pos = _positions(pmode, B, Tq, N, m, g)
    I = torch.full((B, Tq, N), float("nan"), dtype=torch.float32, device=DEV)
    csa.csa_index_score(qI, w, K, pos, I, m=m, K_scale=Ks)
    torch.cuda.synchronize()
    got = to_f64(I)
    for b in range(B):
        Kb = to_f64(K[b]) * (to_f64(Ks[b])[:, None] if Ks is not None else 1.0)
        ref = O.index_score(to_f64(qI[b]), to_f64(w[b]), Kb, to_f64(pos[b]), m=m)
        assert np.array_equal(np.isneginf(got[b]), np.isneginf(ref)), name
        fin = np.isfinite(ref)
        assert np.all(np.isfinite(got[b][fin]))
        err = row_rel_err(np.where(fin, got[b], 0.0), np.where(fin, ref, 0.0))
        assert err <= TOL_F32, (name, b, err)


# ---------------------------------------------------------------------------
# a3 top-k (bit-exact)
# ---------------------------------------------------------------------------
TOPK_CASES = [
    # name, B, Tq, N, m, k, score kind, positions
    ("normal_single_stage", 2, 7, 3000, 4, 16, "normal", "partial"),
    ("heavy_ties_zeros", 1, 9, 2500, 1, 512, "ties", "partial"),
    ("k_exceeds_visible", 1, 4, 600, 4, 2048, "ties", "partial"),
    ("k1_and_pow2_edges", 2, 3, 1025, 1, 1, "normal", "all"),
    ("two_stage_decode", 3, 1, 70000, 4, 1024, "normal", "partial"),
    ("two_stage_ties", 2, 1, 40000, 1, 1024, "ties", "all"),
    ("two_stage_k512_flash_like", 2, 1, 16384, 4, 512, "normal", "all"),
    ("prefill_rows", 1, 600, 2000, 4, 1024, "normal", "prefill"),
    ("decode_1M_full_shape", 16, 1, 262144, 4, 1024, "normal", "all"),
    ("prefill_full_row_length", 1, 40, 32768, 4, 1024, "normal", "prefill"),
]


def _scores(g, kind, shape):
    x = g.normal(1, shape, "f32")
    if kind == "ties":
        x = torch.floor(x * 2.0) / 2.0                 # few distinct values
        x[..., ::7] = 0.0
        x[..., 3::7] = -0.0
    return x.contiguous()


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk_bit_exact(csa, case):
    name, B, Tq, N, m, k, kind, pmode = case
    g = Gen(300 + TOPK_CASES.index(case), DEV)
    I = _scores(g, kind, (B, Tq, N))
    pos = _positions(pmode, B, Tq, N, m, g)
    ws_n = csa.csa_topk_workspace_size(B, Tq, N, k)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=DEV)
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=DEV)
    val = torch.empty((B, Tq, k), dtype=torch.float32, device=DEV)
    csa.csa_topk(I, pos, idx, m=m, k=k, val_out=val, workspace=ws)
    torch.cuda.synchronize()
    got_i = idx.cpu().numpy()
    got_v = val.cpu().numpy()
    In = I.cpu().numpy()
    for b in range(B):
        ref_i, _ = O.topk(In[b].astype(np.float64), pos[b].cpu().numpy(), m=m, k=k)
        assert np.array_equal(got_i[b], ref_i), (name, b)
        sel = ref_i >= 0
        exp_v = np.where(sel, np.take_along_axis(In[b], np.maximum(ref_i, 0), axis=1), -np.inf)
        assert np.array_equal(got_v[b].view(np.uint32), exp_v.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# a4 / a5 attention
# ---------------------------------------------------------------------------
MQA_CASES = [
    # name, dense, dt, B, Tq, n_h, d, N, k, m, n_win, W_cap, rope, sink, gamma, positions
    ("tiny_f32_sparse", False, "f32", 1, 256, 4, 64, 64, 16, 4, 16, 256, 16, "zero", True, "prefill0"),
    ("f32_dense_hca", True, "f32", 2, 3, 4, 64, 100, 0, 4, 8, 16, 16, "normal", False, "partial"),
    ("bf16_sparse_decode_split", False, "bf16", 3, 1, 64, 512, 900, 512, 4, 128, 128, 64, "normal", True, "all"),
    ("bf16_sparse_decode_h128_k1024", False, "bf16", 2, 1, 128, 512, 3000, 1024, 4, 128, 128, 64, "normal", False, "all"),
    ("bf16_sparse_prefill_nosplit", False, "bf16", 1, 24, 128, 512, 500, 64, 4, 128, 4096, 64, "normal", True, "prefill"),
    ("bf16_dense_decode_split", True, "bf16", 2, 1, 64, 512, 1500, 0, 128, 128, 128, 64, "normal", False, "all"),
    ("bf16_dense_prefill", True, "bf16", 1, 20, 32, 256, 90, 0, 4, 32, 512, 32, "none", True, "prefill"),
    ("bf16_sparse_d128_nowindow", False, "bf16", 2, 2, 16, 128, 200, 40, 4, 0, 0, 128, "none", False, "partial"),
    ("bf16_generic_h8", False, "bf16", 1, 2, 8, 64, 100, 20, 4, 10, 10, 16, "normal", True, "all"),
    ("bf16_decode_one_split_h32_d256", False, "bf16", 2, 3, 32, 256, 300, 100, 4, 64, 64, 32, "normal", True, "partial"),
    ("bf16_decode_dense_h96_d128", True, "bf16", 2, 1, 96, 128, 700, 0, 4, 16, 32, 32, "none", False, "all"),
    # prefill through the streaming kernel: a full 2,048-slot range, then two ranges and a combine
    ("bf16_sparse_prefill_table_full", False, "bf16", 1, 16, 32, 128, 3000, 2000, 4, 48, 64, 32, "none", False, "all"),
    ("bf16_dense_prefill_two_ranges", True, "bf16", 1, 16, 32, 128, 2300, 0, 4, 64, 128, 32, "normal", True, "all"),
]


@pytest.mark.parametrize("case", MQA_CASES, ids=[c[0] for c in MQA_CASES])
def test_mqa_parity(csa, case):
    name, dense, dt, B, Tq, n_h, d, N, k, m, n_win, W_cap, rope, sink_kind, use_gamma, pmode = case
    g = Gen(400 + MQA_CASES.index(case), DEV)
    q = g.normal(1, (B, Tq, n_h, d), dt)
    E = g.normal(2, (B, N, d), dt)
    W = g.normal(3, (B, W_cap, d), dt) if n_win > 0 else None
    sink = {"none": None, "zero": torch.zeros(n_h, device=DEV),
            "normal": g.normal(4, (n_h,), "f32", per_slot=False)}[sink_kind]
    gamma = _gamma(g, 5, d) if use_gamma else None
    pos = _positions(pmode, B, Tq, N, m, g)
    out = torch.full_like(q, float("nan"))
    slots = (N if dense else k) + n_win
    ws_n = csa.csa_mqa_workspace_size(B, Tq, n_h, d, slots)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(d)
    if dense:
        csa.hca_dense_mqa(q, E, W, pos, out, m=m, n_win=n_win, sink=sink, gamma_q=gamma, rope_dim=rope,
                          scale=scale, workspace=ws)
    else:
        # slots: distinct entries, with empty (-1) and out-of-range slots mixed in
        u = g.uniform(6, (B, Tq, k))
        idx = (u * (N + 8)).to(torch.int32) - 4
        idx[..., ::5] = -1
        idx = idx.contiguous()
        csa.csa_sparse_mqa(q, E, idx, W, pos, out, n_win=n_win, sink=sink, gamma_q=gamma, rope_dim=rope,
                           scale=scale, workspace=ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    sk = None if sink is None else to_f64(sink)
    gm = None if gamma is None else to_f64(gamma)
    for b in range(B):
        kw = dict(q_pos=to_f64(pos[b]), n_win=n_win, W_cap=W_cap if n_win else None, gamma_q=gm,
                  eps=1e-6, sink=sk, rope_dim=rope, scale=scale)
        Wb = to_f64(W[b]) if W is not None else None
        if dense:
            ref = O.dense_mqa(to_f64(q[b]), to_f64(E[b]), Wb, m=m, **kw)
        else:
            ref = O.sparse_mqa(to_f64(q[b]), to_f64(E[b]), to_f64(idx[b]), Wb, **kw)
        err = row_rel_err(got[b], ref)
        assert err <= tol, (name, b, err)


def test_mqa_empty_key_set_is_zero(csa):
    """k slots all empty, no window, no sink: the output row is 0 (both paths)."""
    for dt, d, n_h in (("bf16", 128, 16), ("bf16", 512, 32), ("f32", 64, 4)):
        g = Gen(480, DEV)
        q = g.normal(1, (1, 2, n_h, d), dt)
        E = g.normal(2, (1, 10, d), dt)
        idx = torch.full((1, 2, 4), -1, dtype=torch.int32, device=DEV)
        pos = torch.tensor([[50, 60]], dtype=torch.int32, device=DEV)
        out = torch.full_like(q, float("nan"))
        csa.csa_sparse_mqa(q, E, idx, None, pos, out, n_win=0, rope_dim=16)
        torch.cuda.synchronize()
        assert torch.all(out == 0), dt


def test_mqa_split_partials_large_values(csa):
    """A split decode query whose entries reach about +-4.5e4: the split partials
    (each split's output divided by its softmax sum, kept as fp16) stay inside the
    fp16 range, and the merged rows match the oracle to the bf16 tolerance.  Large
    entries also make the softmax close to one-hot, the case where a partial row
    is as large as the largest value row."""
    B, Tq, n_h, d, N, k, m, n_win, rope = 2, 1, 64, 512, 900, 512, 4, 128, 64
    g = Gen(490, DEV)
    q = g.normal(1, (B, Tq, n_h, d), "bf16")
    E = (g.normal(2, (B, N, d), "f32") * 1e4).to(torch.bfloat16)
    W = (g.normal(3, (B, n_win, d), "f32") * 1e4).to(torch.bfloat16)
    sink = g.normal(4, (n_h,), "f32", per_slot=False)
    pos = _positions("all", B, Tq, N, m, g)
    idx = ((g.uniform(6, (B, Tq, k)) * N).to(torch.int32)).contiguous()
    ws = torch.empty(csa.csa_mqa_workspace_size(B, Tq, n_h, d, k + n_win), dtype=torch.uint8, device=DEV)
    assert ws.numel() > 0   # the query is split
    out = torch.full_like(q, float("nan"))
    scale = 1.0 / math.sqrt(d)
    csa.csa_sparse_mqa(q, E, idx, W, pos, out, n_win=n_win, sink=sink, rope_dim=rope, scale=scale,
                       workspace=ws)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.isfinite(got).all()
    for b in range(B):
        ref = O.sparse_mqa(to_f64(q[b]), to_f64(E[b]), to_f64(idx[b]), to_f64(W[b]), q_pos=to_f64(pos[b]),
                           n_win=n_win, W_cap=n_win, gamma_q=None, eps=1e-6, sink=to_f64(sink),
                           rope_dim=rope, scale=scale)
        assert np.abs(ref).max() > 3e4
        err = row_rel_err(got[b], ref)
        assert err <= TOL_BF16, (b, err)


def test_mqa_unaligned_output_takes_generic_path(csa):
    """A bf16 call whose output is not 16-byte aligned (a view 2 bytes into its
    buffer) takes the generic kernel; it still matches the oracle, and leaves
    the element before the view untouched."""
    B, Tq, n_h, d, N, k, m, n_win, rope = 1, 2, 16, 128, 200, 40, 4, 16, 32
    g = Gen(495, DEV)
    q = g.normal(1, (B, Tq, n_h, d), "bf16")
    E = g.normal(2, (B, N, d), "bf16")
    W = g.normal(3, (B, n_win, d), "bf16")
    pos = _positions("all", B, Tq, N, m, g)
    idx = ((g.uniform(6, (B, Tq, k)) * N).to(torch.int32)).contiguous()
    n = B * Tq * n_h * d
    buf = torch.full((n + 8,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[1:1 + n].view(B, Tq, n_h, d)
    assert out.data_ptr() % 16 != 0
    ws = torch.empty(max(1, csa.csa_mqa_workspace_size(B, Tq, n_h, d, k + n_win)), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(d)
    csa.csa_sparse_mqa(q, E, idx, W, pos, out, n_win=n_win, rope_dim=rope, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    assert float(buf[0]) == 7.0 and float(buf[n + 1]) == 7.0
    got = to_f64(out)
    for b in range(B):
        ref = O.sparse_mqa(to_f64(q[b]), to_f64(E[b]), to_f64(idx[b]), to_f64(W[b]), q_pos=to_f64(pos[b]),
                           n_win=n_win, W_cap=n_win, gamma_q=None, eps=1e-6, sink=None, rope_dim=rope,
                           scale=scale)
        assert row_rel_err(got[b], ref) <= TOL_BF16
