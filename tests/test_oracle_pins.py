"""Pins of the fp64 oracle against facts that do not come from the oracle:
closed forms, invariants, special cases that reduce to library routines,
brute-force ranking on tiny inputs and hand-derived fixtures.

Each group names the property of the pages it checks.  A plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand, a
wrong block boundary) fails at least one of them; see the
``test_planted_mistakes_are_caught`` group at the end, which plants such
mistakes in copies of oracle functions and checks that the pins notice.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs as oc
from oracle import csa as O

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------------------
# codecs: against the format definitions and torch's own conversions
# ---------------------------------------------------------------------------
def test_bf16_decode_all_codes_match_torch():
    codes = np.arange(65536, dtype=np.uint16)
    ours = oc.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_decode_all_codes_match_torch_and_closed_form():
    codes = np.arange(256, dtype=np.uint8)
    ours = oc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0
    assert ours[0x80] == 0.0 and math.copysign(1, ours[0x80]) == -1


def test_bf16_rne_matches_torch_and_ties():
    x = RNG.standard_normal(20000).astype(np.float32) * np.float32(1e3)
    ours = oc.f64_to_bf16_value(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oc.f64_to_bf16_value(1 + 2.0 ** -8) == 1.0
    assert oc.f64_to_bf16_value(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert oc.f64_to_bf16_value(2.0 ** -133) == 2.0 ** -133          # smallest subnormal
    assert oc.f64_to_bf16_value(2.0 ** -134) == 0.0                   # tie to even (0)


def test_e4m3_rne_sat_matches_torch_and_ties():
    x = (RNG.standard_normal(20000) * 60).astype(np.float32)
    x = np.clip(x, -448, 448)
    ours = oc.f64_to_e4m3_value(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(ours, ref)
    assert oc.f64_to_e4m3_value(1 + 1 / 16) == 1.0
    assert oc.f64_to_e4m3_value(1 + 3 / 16) == 1.25
    assert oc.f64_to_e4m3_value(500.0) == 448.0 and oc.f64_to_e4m3_value(-1e9) == -448.0
    assert oc.f64_to_e4m3_value(2.0 ** -10) == 0.0                    # half the min subnormal
    assert oc.f64_to_e4m3_value(3 * 2.0 ** -10) == 2.0 ** -8
    assert np.array_equal(oc.e4m3_code([1.0, -448.0, 2.0 ** -9]), [0x38, 0xFE, 0x01])


def test_oracle_fp8_row_quantisation_is_faithful():
    E = RNG.standard_normal((5, 128))
    E[2] = 0.0
    codes, scale = O.quantize_rows_e4m3(E)
    assert scale[2] == 1.0 and np.all(codes[2] == 0)
    dec = oc.e4m3_to_f64(codes) * scale[:, None].astype(np.float64)
    # |error| <= half an e4m3 ulp at the element's binade (relative 2^-4), plus subnormal slack
    err = np.abs(dec - E)
    bound = np.maximum(np.abs(E) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * 1.0001
    assert np.all(err <= bound)
    # the row maximum maps to +-448 exactly
    j = np.argmax(np.abs(E[0]))
    assert abs(oc.e4m3_to_f64(codes[0, j])) == 448.0


# ---------------------------------------------------------------------------
# a1 compressor: geometry, convexity, closed forms
# ---------------------------------------------------------------------------
def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_compress_golden_geometry(golden_dir):
    g = _load(golden_dir, "compress_geometry.json")
    T = g["T"]
    Ca = np.array(g["C_a"], dtype=np.float64)[:, None]
    Cb = np.array(g["C_b"], dtype=np.float64)[:, None]
    for case in g["cases"]:
        E = O.pool_entries(Ca, None, Cb, None, m=case["m"], overlap=case["overlap"], T=T)
        assert E.shape == (len(case["expected"]), 1)
        assert np.allclose(E[:, 0], case["expected"], rtol=0, atol=1e-12), case


@pytest.mark.parametrize("T,m,n", [(256, 4, 64), (257, 4, 65), (255, 4, 64), (1, 4, 1),
                                   (1048576, 128, 8192), (1048577, 128, 8193)])
def test_entry_count_is_ceil(T, m, n):
    assert O.num_entries(T, m) == n


def test_entry_count_from_pooling():
    c = 3
    for T in (256, 257):
        C = RNG.standard_normal((T, c))
        E = O.pool_entries(C, C, C, C, m=4, overlap=1, T=T)
        assert E.shape[0] == math.ceil(T / 4)


def test_each_token_feeds_exactly_two_entries():
    # count candidate memberships from the candidate sets themselves
    T, m = 37, 4
    hits = np.zeros(T, dtype=int)
    for s in range(O.num_entries(T, m)):
        for _, t in O.candidate_tokens(s, m, 1, T):
            hits[t] += 1
    # every token but those of the last (partial) block feeds two entries
    last_block_start = m * (O.num_entries(T, m) - 1)
    assert np.all(hits[:last_block_start] == 2)
    assert np.all(hits[last_block_start:] == 1)


def test_constant_rows_pool_to_constant():
    T, c = 23, 5
    v = RNG.standard_normal(c)
    C = np.tile(v, (T, 1))
    Za, Zb = RNG.standard_normal((T, c)) * 5, RNG.standard_normal((T, c)) * 5
    for m, ov in ((4, 1), (4, 0), (8, 1), (128, 0)):
        E = O.pool_entries(C, Za, C, Zb, m=m, overlap=ov, T=T)
        assert np.allclose(E, v, atol=1e-13)


def test_dominant_logit_selects_previous_block_candidate():
    # C_b / Z_b of token tau feed entry tau//m + 1 (the "previous block" set)
    T, m, c = 24, 4, 3
    for tau in (0, 5, 11, 19):
        Ca = np.zeros((T, c)); Cb = np.zeros((T, c))
        Za = np.zeros((T, c)); Zb = np.zeros((T, c))
        Cb[tau] = [1.0, 2.0, 3.0]
        Zb[tau] = 50.0
        E = O.pool_entries(Ca, Za, Cb, Zb, m=m, overlap=1, T=T)
        s = tau // m + 1
        assert np.allclose(E[s], [1.0, 2.0, 3.0], rtol=1e-15, atol=1e-17 * 1e3 + 1e-20)
        others = np.delete(E, s, axis=0)
        assert np.all(others == 0.0)


def test_dominant_logit_selects_own_block_candidate():
    T, m, c = 24, 4, 2
    tau = 9
    Ca = RNG.standard_normal((T, c)); Cb = RNG.standard_normal((T, c))
    Za = np.zeros((T, c)); Zb = np.zeros((T, c))
    Za[tau] = 60.0
    E = O.pool_entries(Ca, Za, Cb, Zb, m=m, overlap=1, T=T)
    assert np.allclose(E[tau // m], Ca[tau], atol=1e-20 + 1e-12)


def test_identity_at_m1_without_overlap():
    T, c = 17, 6
    C = RNG.standard_normal((T, c))
    Z = RNG.standard_normal((T, c)) * 10
    E = O.pool_entries(C, Z, None, None, m=1, overlap=0, T=T)
    assert np.array_equal(E, C)


def test_channels_independent_and_linear_in_C():
    T, c, m = 30, 7, 4
    Ca, Cb = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    Za, Zb = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    E = O.pool_entries(Ca, Za, Cb, Zb, m=m, overlap=1, T=T)
    perm = RNG.permutation(c)
    Ep = O.pool_entries(Ca[:, perm], Za[:, perm], Cb[:, perm], Zb[:, perm], m=m, overlap=1, T=T)
    assert np.allclose(Ep, E[:, perm], atol=1e-14)
    Ca2, Cb2 = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    E2 = O.pool_entries(Ca2, Za, Cb2, Zb, m=m, overlap=1, T=T)
    E3 = O.pool_entries(2 * Ca - 3 * Ca2, Za, 2 * Cb - 3 * Cb2, Zb, m=m, overlap=1, T=T)
    assert np.allclose(E3, 2 * E - 3 * E2, atol=1e-12)


def test_logit_shift_invariance():
    # a softmax is unchanged by adding a per-channel constant to all of one entry's logits
    T, c, m = 16, 4, 4
    Ca, Cb = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    Z = RNG.standard_normal((T, c))
    E = O.pool_entries(Ca, Z, Cb, Z, m=m, overlap=1, T=T)
    E2 = O.pool_entries(Ca, Z + 7.5, Cb, Z + 7.5, m=m, overlap=1, T=T)
    assert np.allclose(E, E2, atol=1e-13)


def test_tok_base_window_of_rows():
    # compressing from a slice of rows equals compressing from all rows
    T, c, m = 40, 3, 4
    Ca, Cb = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    Za, Zb = RNG.standard_normal((T, c)), RNG.standard_normal((T, c))
    full = O.pool_entries(Ca, Za, Cb, Zb, m=m, overlap=1, T=T)
    base = 4 * 6 - 4
    part = O.pool_entries(Ca[base:], Za[base:], Cb[base:], Zb[base:], m=m, overlap=1, T=T,
                          tok_base=base, s_begin=6, s_end=10)
    assert np.array_equal(part, full[6:10])
    with pytest.raises(ValueError):
        O.pool_entries(Ca[base + 1:], Za[base + 1:], Cb[base + 1:], Zb[base + 1:], m=m,
                       overlap=1, T=T, tok_base=base + 1, s_begin=6, s_end=7)


# ---------------------------------------------------------------------------
# RMSNorm and RoPE
# ---------------------------------------------------------------------------
def test_rmsnorm_closed_form():
    x = RNG.standard_normal((9, 64)) * 3
    eps = 1e-3
    y = O.rmsnorm(x, None, eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13)
    assert np.allclose(O.rmsnorm(5.0 * x, None, 0.0), O.rmsnorm(x, None, 0.0), rtol=1e-13)
    g = RNG.standard_normal(64)
    assert np.allclose(O.rmsnorm(x, g, eps), y * g, rtol=1e-14)
    assert np.all(O.rmsnorm(np.zeros((1, 8)), None, 1e-6) == 0)


def test_rope_closed_forms():
    # r = 2: theta_0 = base^0 = 1, pair (1, 0) at position 1 -> (cos 1, sin 1)
    x = np.array([5.0, 1.0, 0.0])
    y = O.rope(x, 1, 2)
    assert y[0] == 5.0 and np.allclose(y[1:], [math.cos(1), math.sin(1)], rtol=1e-15)
    # r = 4, base 10000: theta_1 = 10000^(-1/2) = 0.01; at p = 100 the second pair turns by 1 rad
    x = np.array([0.0, 0.0, 1.0, 0.0])
    y = O.rope(x, 100, 4, 10000.0)
    assert np.allclose(y, [0.0, 0.0, math.cos(1), math.sin(1)], atol=1e-12)
    x = np.array([1.0, 0.0, 0.0, 0.0])
    assert np.allclose(O.rope(x, 100, 4, 10000.0), [math.cos(100), math.sin(100), 0, 0], atol=1e-12)


def test_rope_group_properties():
    x = RNG.standard_normal((6, 64))
    r = 16
    for p in (0, 3, 1000, 1048576):
        y = O.rope(x, p, r)
        assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
        assert np.array_equal(y[:, : 64 - r], x[:, : 64 - r])
    assert np.allclose(O.rope(x, 0, r), x, atol=0)
    assert np.allclose(O.rope(O.rope(x, 17, r), 25, r), O.rope(x, 42, r), atol=1e-12)
    assert np.allclose(O.rope(O.rope(x, 77, r), -77, r), x, atol=1e-12)
    # relative: <R_i q, R_j k> depends only on i - j
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    a = O.rope(q, 10, r) @ O.rope(k, 3, r)
    b = O.rope(q, 1010, r) @ O.rope(k, 1003, r)
    assert np.isclose(a, b, rtol=1e-11)


def test_compress_applies_norm_then_rope_at_block_start():
    T, c, m, r = 16, 8, 4, 4
    C = RNG.standard_normal((T, c))
    E = O.compress(C, None, C, None, m=m, overlap=0, T=T, rope_dim=r, eps=0.0)
    pooled = np.stack([C[m * s:m * s + m].mean(axis=0) for s in range(T // m)])
    normed = pooled / np.sqrt(np.mean(pooled ** 2, axis=-1, keepdims=True))
    for s in range(T // m):
        assert np.allclose(O.rope(E[s], -m * s, r), normed[s], atol=1e-13)


# ---------------------------------------------------------------------------
# a2 indexer score
# ---------------------------------------------------------------------------
def test_index_score_scaled_keys_are_linear_in_index():
    Tq, H, dI, N, m = 3, 5, 8, 40, 1
    q = RNG.standard_normal((Tq, H, dI))
    w = RNG.uniform(size=(Tq, H))
    v = RNG.standard_normal(dI)
    K = np.arange(N)[:, None] * v[None, :]          # K_s = s * v
    I = O.index_score(q, w, K, [N - 1] * Tq, m=m)
    ref = np.array([np.sum(w[t] * np.maximum(q[t] @ v, 0)) for t in range(Tq)])
    assert np.allclose(I, np.arange(N)[None, :] * ref[:, None], rtol=1e-13)


def test_index_score_relu_sign_and_weights():
    H, dI = 4, 16
    v = RNG.standard_normal(dI)
    K = np.tile(v, (6, 1))
    w = RNG.uniform(size=(1, H))
    q_pos_all = [5]
    I_neg = O.index_score(-np.tile(v, (1, H, 1)), w, K, q_pos_all, m=1)
    assert np.all(I_neg == 0.0)
    I_pos = O.index_score(np.tile(v, (1, H, 1)), w, K, q_pos_all, m=1)
    assert np.allclose(I_pos, w.sum() * (v @ v), rtol=1e-13)
    # mixed: head 0 positive, others negative -> only w0 * |v|^2 survives
    q = -np.tile(v, (1, H, 1)); q[0, 0] = v
    assert np.allclose(O.index_score(q, w, K, q_pos_all, m=1), w[0, 0] * (v @ v), rtol=1e-13)


def test_index_score_visibility_rule_and_mask():
    Tq, H, dI, N, m = 20, 2, 4, 6, 4
    q = RNG.standard_normal((Tq, H, dI)); w = RNG.uniform(size=(Tq, H))
    K = RNG.standard_normal((N, dI))
    pos = np.arange(Tq)
    I = O.index_score(q, w, K, pos, m=m)
    for t, i in enumerate(pos):
        finite = np.isfinite(I[t])
        n = min(N, (i + 1) // m)
        assert finite.sum() == n and np.all(finite[:n])
        assert np.all(I[t, n:] == -np.inf)
        # entry s is visible iff all its tokens m s .. m s + m - 1 are <= i
        for s in range(N):
            assert finite[s] == (m * s + m - 1 <= i)
    assert np.all(I[np.isfinite(I)] >= 0)                    # w >= 0 -> I >= 0


def test_index_score_positive_homogeneity_in_key_scale():
    q = RNG.standard_normal((2, 3, 8)); w = RNG.standard_normal((2, 3))
    K = RNG.standard_normal((10, 8))
    scales = RNG.uniform(0.1, 3.0, size=10)
    I1 = O.index_score(q, w, K * scales[:, None], [39, 39], m=4)
    I2 = O.index_score(q, w, K, [39, 39], m=4) * scales[None, :]
    assert np.allclose(I1, I2, rtol=1e-12)


# ---------------------------------------------------------------------------
# a3 top-k
# ---------------------------------------------------------------------------
def test_topk_golden_ties(golden_dir):
    g = _load(golden_dir, "topk_ties.json")
    s = np.array([float(v) for v in g["scores"]])
    assert math.copysign(1, s[4]) == -1
    for case in g["cases"]:
        idx, vals = O.topk(s[None, :], [g["q_pos"]], m=g["m"], k=case["k"])
        assert list(idx[0]) == case["expected"], case


def _rank_select(scores, k):
    """Brute force by counting: element s is beaten by s' if it scores more,
    or the same with a lower index; keep the k least beaten."""
    n = len(scores)
    beaten = [sum(1 for j in range(n) if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
              for i in range(n)]
    order = sorted(range(n), key=lambda i: beaten[i])
    return order[:min(k, n)]


def test_topk_exhaustive_tiny_against_rank_counting():
    vals = [-1.0, 0.0, -0.0, 1.0, 2.0]
    rng = np.random.default_rng(7)
    for n in range(1, 8):
        for trial in range(40):
            row = rng.choice(vals, size=n)
            for k in range(1, n + 2):
                idx, _ = O.topk(row[None, :], [n - 1], m=1, k=k)
                exp = _rank_select(list(row), k)
                assert list(idx[0, :len(exp)]) == exp
                assert np.all(idx[0, len(exp):] == -1)


def test_topk_respects_visibility():
    N, m = 50, 4
    row = RNG.standard_normal(N)
    row[40:] = 1e9                                       # huge but invisible scores
    idx, _ = O.topk(row[None, :], [4 * 10 - 1], m=m, k=100)
    assert set(idx[0][idx[0] >= 0]) == set(range(10))
    assert np.sum(idx[0] >= 0) == 10


# ---------------------------------------------------------------------------
# a4 / a5 attention
# ---------------------------------------------------------------------------
def test_sink_closed_forms(golden_dir):
    g = _load(golden_dir, "attention_sink.json")
    q = np.array([g["q"]]); kv = np.array(g["kv"])
    for case in g["cases"]:
        KV = np.tile(kv, (case["n"], 1))
        sig = float(case["sigma"])
        o = O.attend_one(q, KV, i=0, eps=0.0, sink=[sig], scale=g["scale"])
        assert np.allclose(o[0], kv * case["weight"], rtol=1e-14), case


def test_no_keys_no_sink_is_zero_and_sink_only_is_zero():
    q = RNG.standard_normal((2, 8))
    assert np.all(O.attend_one(q, np.zeros((0, 8)), i=3, sink=None, scale=0.3) == 0)
    assert np.all(O.attend_one(q, np.zeros((0, 8)), i=3, sink=[0.5, -1.0], scale=0.3) == 0)


def test_csa_special_case_equals_textbook_causal_attention():
    """m = 1 without overlap (entries = normalised raw rows), k >= n, no window,
    no sink, no RoPE: CSA is textbook causal softmax attention with K = V."""
    T, n_h, d, H, dI = 24, 3, 16, 2, 8
    raw = RNG.standard_normal((T, d))
    E = O.compress(raw, None, None, None, m=1, overlap=0, T=T, rope_dim=0, eps=1e-6)
    q = RNG.standard_normal((T, n_h, d))
    qI = RNG.standard_normal((T, H, dI)); w = RNG.uniform(size=(T, H))
    KI = RNG.standard_normal((T, dI))
    pos = np.arange(T)
    I = O.index_score(qI, w, KI, pos, m=1)
    idx, _ = O.topk(I, pos, m=1, k=T)
    out = O.sparse_mqa(q, E, idx, None, q_pos=pos, n_win=0, eps=1e-6, sink=None,
                       rope_dim=0, scale=1 / math.sqrt(d))
    qh = torch.from_numpy(O.rmsnorm(q, None, 1e-6)).permute(1, 0, 2)      # [n_h, T, d]
    kv = torch.from_numpy(E)[None].expand(n_h, T, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kv, kv, is_causal=True)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_sparse_with_all_entries_equals_dense():
    T, n_h, d, m, r = 40, 2, 16, 4, 4
    E = RNG.standard_normal((T // m, d)); W = RNG.standard_normal((64, d))
    q = RNG.standard_normal((T, n_h, d)); sink = RNG.standard_normal(n_h)
    pos = np.arange(T)
    idx = np.array([[s if s < (i + 1) // m else -1 for s in range(T // m)] for i in pos])
    a = O.sparse_mqa(q, E, idx, W, q_pos=pos, n_win=8, sink=sink, rope_dim=r, scale=0.25)
    b = O.dense_mqa(q, E, W, q_pos=pos, m=m, n_win=8, sink=sink, rope_dim=r, scale=0.25)
    assert np.allclose(a, b, atol=1e-14)


def test_constant_values_give_value_times_total_weight():
    n_h, d, r, i = 3, 16, 4, 57
    v = RNG.standard_normal(d)
    KV = np.tile(v, (9, 1))
    q = RNG.standard_normal((n_h, d)); sink = RNG.standard_normal(n_h)
    scale = 0.2
    o = O.attend_one(q, KV, i=i, sink=sink, rope_dim=r, scale=scale)
    qh = O.rope(O.rmsnorm(q, None, 1e-6), i, r)
    for h in range(n_h):
        l = scale * qh[h] @ v
        p = 9 * math.exp(l) / (9 * math.exp(l) + math.exp(sink[h]))
        assert np.allclose(o[h], O.rope(p * v, -i, r), rtol=1e-12, atol=1e-14)
        assert p < 1


def test_window_extent_and_ring_rows():
    # one-hot rows mark which tokens enter the window; q = 0 makes logits equal
    d, n_win, W_cap = 64, 5, 16
    W = np.zeros((W_cap, d))
    for row in range(W_cap):
        W[row, row] = 1.0
    q = np.zeros((1, 1, d))
    for i in (0, 3, 4, 20, 35):
        out = O.sparse_mqa(q, np.zeros((1, d)), np.array([[-1]]), W, q_pos=[i], n_win=n_win,
                           W_cap=W_cap, eps=1.0, rope_dim=0, scale=1.0)
        toks = list(range(max(0, i - n_win + 1), i + 1))
        exp = np.zeros(d)
        for t in toks:
            exp[t % W_cap] += 1.0 / len(toks)
        assert np.allclose(out[0, 0], exp, atol=1e-15)


def test_idx_permutation_invariance():
    d, n_h = 32, 2
    E = RNG.standard_normal((30, d)); W = RNG.standard_normal((8, d))
    q = RNG.standard_normal((1, n_h, d))
    idx = np.array([[3, 17, 5, 29, -1, 0]])
    a = O.sparse_mqa(q, E, idx, W, q_pos=[200], n_win=4, W_cap=8, sink=[0.1, -0.3],
                     rope_dim=8, scale=0.2)
    b = O.sparse_mqa(q, E, idx[:, ::-1].copy(), W, q_pos=[200], n_win=4, W_cap=8,
                     sink=[0.1, -0.3], rope_dim=8, scale=0.2)
    assert np.allclose(a, b, atol=1e-14)


def test_shift_invariance_needs_output_rotation_at_minus_i():
    """Shifting the query, every entry and every window token by D leaves the
    de-rotated output unchanged (the output is rotated again at -i)."""
    d, r, n_h, m = 32, 8, 2, 4
    raw_E = RNG.standard_normal((12, d)); raw_W = RNG.standard_normal((16, d))
    q = RNG.standard_normal((1, n_h, d)); sink = RNG.standard_normal(n_h)
    i = 50
    idx = np.array([[0, 3, 7, 11]])

    def run(D):
        E = np.stack([O.rope(raw_E[s], m * s + D, r) for s in range(12)])
        W = np.zeros((16 + 64, d))
        for tau in range(i - 15, i + 1):
            W[(tau + D) % 80] = O.rope(raw_W[tau - (i - 15)], tau + D, r)
        return O.sparse_mqa(q, E, idx, W, q_pos=[i + D], n_win=16, W_cap=80, sink=sink,
                            rope_dim=r, scale=0.2)

    a, b = run(0), run(12345)
    assert np.allclose(a, b, rtol=1e-9, atol=1e-11)
    assert not np.allclose(O.rope(a, 7, r), a)   # the rotation is not trivial here


# ---------------------------------------------------------------------------
# planted mistakes: the pins above must notice plausible oracle bugs
# ---------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch, golden_dir):
    g = _load(golden_dir, "compress_geometry.json")
    T = g["T"]
    Ca = np.array(g["C_a"], dtype=np.float64)[:, None]
    Cb = np.array(g["C_b"], dtype=np.float64)[:, None]

    # (1) wrong block for set b: the next block instead of the previous one
    def bad_candidates(s, m, overlap, T):
        a = [("a", t) for t in range(m * s, min(m * (s + 1), T))]
        b = [("b", t) for t in range(m * (s + 1), min(m * (s + 2), T))] if overlap else []
        return a + b
    with monkeypatch.context() as mp:
        mp.setattr(O, "candidate_tokens", bad_candidates)
        E = O.pool_entries(Ca, None, Cb, None, m=4, overlap=1, T=T)
        assert not np.allclose(E[:, 0], g["cases"][0]["expected"])

    # (2) visibility off by one (a query seeing its own block)
    with monkeypatch.context() as mp:
        mp.setattr(O, "n_visible", lambda i, m, N: min(N, i // m + 1))
        I = O.index_score(np.ones((1, 1, 2)), np.ones((1, 1)), np.ones((4, 2)), [5], m=4)
        assert np.isfinite(I[0]).sum() != 1           # the pin expects floor(6/4) = 1

    # (3) output rotated at +i instead of -i breaks shift invariance
    real_rope = O.rope

    def attend_wrong_sign(q, KV, *, i, **kw):
        out = O_attend_orig(q, KV, i=i, **kw)
        r = kw.get("rope_dim", 0)
        return real_rope(real_rope(out, i, r), i, r)  # = rotated at +i overall
    O_attend_orig = O.attend_one
    with monkeypatch.context() as mp:
        mp.setattr(O, "attend_one", attend_wrong_sign)
        with pytest.raises(AssertionError):
            test_shift_invariance_needs_output_rotation_at_minus_i()

    # (4) sink added to the numerator too (total weight 1) breaks the closed form
    def attend_sink_as_key(q, KV, *, i, sink=None, **kw):
        return O_attend_orig(q, KV, i=i, sink=None, **kw)
    with monkeypatch.context() as mp:
        mp.setattr(O, "attend_one", attend_sink_as_key)
        with pytest.raises(AssertionError):
            test_sink_closed_forms(golden_dir)


def test_chunked_prefill_equals_whole_sequence():
    """Chunked-prefill equivalence: the composition that takes cached entries
    for the blocks before the chunk and compresses the rest must give, for every
    chunk query, what the whole-sequence chain (compress all tokens, score,
    select, attend) gives.  Pins the composition's offsets (s0, tok_base,
    window rows) against the plain chain."""
    from oracle import steps
    rng = np.random.default_rng(7)
    T, m, c, dI, H, n_h, k, n_win, r = 96, 4, 16, 8, 2, 3, 5, 6, 4
    p0 = 48
    C = {n: rng.standard_normal((T, c)) for n in ("Ca", "Za", "Cb", "Zb")}
    IC = {n: rng.standard_normal((T, dI)) for n in ("ICa", "IZa", "ICb", "IZb")}
    win_raw = rng.standard_normal((T, c))
    qI = rng.standard_normal((T, H, dI))
    w = rng.uniform(size=(T, H))
    q = rng.standard_normal((T, n_h, c))
    sink = rng.standard_normal(n_h)
    N = T // m
    eps, scale, base = 1e-6, 1 / np.sqrt(c), 10000.0
    # whole sequence
    E = O.compress(C["Ca"], C["Za"], C["Cb"], C["Zb"], m=m, overlap=1, T=T, eps=eps, rope_dim=r)
    K = O.compress(IC["ICa"], IC["IZa"], IC["ICb"], IC["IZb"], m=m, overlap=1, T=T, normalize=False)
    W = O.compress(win_raw, None, None, None, m=1, overlap=0, T=T, eps=eps, rope_dim=r, pos_stride=1)
    pos = np.arange(p0, T)
    I = O.index_score(qI[p0:], w[p0:], K, pos, m=m)
    idx, _ = O.topk(I, pos, m=m, k=k)
    out = O.sparse_mqa(q[p0:], E, idx, W, q_pos=pos, n_win=n_win, eps=eps, sink=sink, rope_dim=r,
                       rope_base=base, scale=scale)
    # chunked: entries before the chunk from the cache (pre-norm pooled rows), the rest compressed
    s0 = p0 // m
    pre = O.pool_entries(C["Ca"], C["Za"], C["Cb"], C["Zb"], m=m, overlap=1, T=T, s_begin=0, s_end=s0)
    KI = np.zeros((N, dI))
    KI[:s0] = K[:s0]
    tb = m * (s0 - 1)
    p = dict(p0=p0, Tq=T - p0, m=m, N=N, k=k, n_win=n_win, rope_dim=r, rope_base=base, eps=eps,
             scale=scale, dtype="f32", k_dtype="f32", KI=KI, tok_base=tb,
             **{n: v[tb:] for n, v in C.items()}, **{n: v[tb:] for n, v in IC.items()},
             win_before=win_raw[p0 - n_win + 1:p0], chunk_raw=win_raw[p0:],
             qI=qI[p0:], w=w[p0:], q=q[p0:], sink=sink)
    ts = np.arange(T - p0)
    got = steps.csa_prefill_queries(p, ts, lambda s: pre[np.asarray(s)])
    np.testing.assert_allclose(got["I"], I, rtol=1e-12, atol=1e-12)
    assert np.array_equal(got["idx"], idx)
    np.testing.assert_allclose(got["out"], out, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# decode compositions (oracle.steps) against the plain whole-sequence chain
# ---------------------------------------------------------------------------
def _store_like(x, dtype, rope_dim=0):
    from oracle.codecs import f64_to_bf16_value
    if dtype == "mixed":
        return O.quantize_rows_mixed(x, rope_dim)[0]
    return f64_to_bf16_value(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def _csa_decode_pin(steps_mod, dtype="bf16", k_dtype="e4m3", with_gamma=False):
    """One CSA decode step (query at i = m N, cached tokens 0 .. i-1) against the
    plain chain over the whole sequence: compress every entry from all tokens,
    store, score, select, attend.  The step's cache rows for entries < N-1 are
    the pooled pre-norm rows (what an earlier step compressed); entry N-1 is
    stale in the cache (its last token just arrived) and must come from the
    step's own compression of tokens m(N-2) .. mN-1 [V4-abs §3.3 compressor
    geometry; §3.5: the state cache holds the tail until its block completes]."""
    from oracle.codecs import e4m3_to_f64
    rng = np.random.default_rng(11)
    m, N, c, dI, H, n_h, k, n_win, r = 4, 24, 16, 8, 3, 2, 7, 6, 4
    if k_dtype == "mxfp4":
        dI = 32                       # one MX block per key
    i = m * N
    T = m * N                         # tokens that feed entries; the query's own token is i
    C = {n: rng.standard_normal((T, c)) for n in ("Ca", "Za", "Cb", "Zb")}
    IC = {n: rng.standard_normal((T, dI)) for n in ("ICa", "IZa", "ICb", "IZb")}
    win_raw = rng.standard_normal((i + 1, c))
    qI = rng.standard_normal((H, dI))
    w = rng.uniform(size=H)
    q = rng.standard_normal((n_h, c))
    sink = rng.standard_normal(n_h)
    gamma = 1.0 + 0.25 * rng.standard_normal(c) if with_gamma else None
    eps, scale, base = 1e-6, 1 / np.sqrt(c), 10000.0
    # plain chain
    E = _store_like(O.compress(C["Ca"], C["Za"], C["Cb"], C["Zb"], m=m, overlap=1, T=T, gamma=gamma, eps=eps,
                               rope_dim=r, rope_base=base), dtype, r)
    K = O.compress(IC["ICa"], IC["IZa"], IC["ICb"], IC["IZb"], m=m, overlap=1, T=T, normalize=False)
    if k_dtype == "mxfp4":
        Kc, Ks = O.quantize_rows_mxfp4(K)
    elif k_dtype == "e4m3":
        codes, sc = O.quantize_rows_e4m3(K)
        K = e4m3_to_f64(codes) * sc.astype(np.float64)[:, None]
    else:
        K = _store_like(K, k_dtype)
    W = _store_like(O.compress(win_raw, None, None, None, m=1, overlap=0, T=i + 1, gamma=gamma, eps=eps,
                               rope_dim=r, rope_base=base, pos_stride=1), dtype, r)
    if k_dtype == "mxfp4":
        I = O.index_score_mxfp4(qI[None], w[None], Kc, Ks, [i], m=m)
    else:
        I = O.index_score(qI[None], w[None], K, [i], m=m)
    idx, _ = O.topk(I, [i], m=m, k=k)
    out = O.sparse_mqa(q[None], E, idx, W, q_pos=[i], n_win=n_win, eps=eps, sink=sink, rope_dim=r,
                       rope_base=base, scale=scale)[0]
    # the step: cached rows, a stale newest entry and key, the newest blocks' candidates
    pre = O.pool_entries(C["Ca"], C["Za"], C["Cb"], C["Zb"], m=m, overlap=1, T=T)
    pre[N - 1] = 1e3 * rng.standard_normal(c)        # stale: must not be read
    if k_dtype == "mxfp4":
        KIc, KIs = Kc.copy(), Ks.copy()
        KIc[N - 1], KIs[N - 1] = 7, 140              # stale: replaced by the step's own key
        keys = dict(KI_codes=KIc, KI_scales=KIs)
        K = oc.mx_fp4_to_f64(Kc, Ks)
    else:
        KI = K.copy()
        KI[N - 1] = 1e3 * rng.standard_normal(dI)    # stale: replaced by the step's own key
        keys = dict(KI=KI)
    tb = m * (N - 2)
    p = dict(i=i, m=m, N=N, k=k, n_win=n_win, d_I=dI, rope_dim=r, rope_base=base, eps=eps, scale=scale,
             dtype=dtype, k_dtype=k_dtype, **keys, win_raw=win_raw[i - n_win + 1:],
             **{n: v[tb:] for n, v in C.items()}, **{n: v[tb:] for n, v in IC.items()},
             qI=qI, w=w, q=q, sink=sink)
    if with_gamma:
        p["gamma"] = gamma
    got = steps_mod.csa_decode_sequence(p, lambda s: pre[np.asarray(s)])
    np.testing.assert_allclose(got["I"], I[0], rtol=1e-12, atol=1e-12)
    assert np.array_equal(got["idx"], idx[0])
    assert (N - 1) in set(idx[0].tolist()), "the fixture must select the newest entry"
    np.testing.assert_allclose(got["k_new"], K[N - 1], rtol=0, atol=0)
    np.testing.assert_allclose(got["out"], out, rtol=1e-10, atol=1e-12)


def _hca_decode_pin(steps_mod, dtype="bf16", with_gamma=False):
    """One HCA decode step (m' = 8, query at i = m' N) against the plain chain:
    compress every block of the whole sequence without overlap, then dense
    attention over every visible entry, the window and the sink [V4-abs §3.3:
    HCA is the non-overlapping, dense variant]."""
    rng = np.random.default_rng(12)
    m, N, c, n_h, n_win, r = 8, 12, 16, 3, 9, 4
    i = m * N
    T = m * N
    Cf, Zf = rng.standard_normal((T, c)), rng.standard_normal((T, c))
    win_raw = rng.standard_normal((i + 1, c))
    q = rng.standard_normal((n_h, c))
    sink = rng.standard_normal(n_h)
    gamma = 1.0 + 0.25 * rng.standard_normal(c) if with_gamma else None
    eps, scale, base = 1e-6, 1 / np.sqrt(c), 10000.0
    E = _store_like(O.compress(Cf, Zf, None, None, m=m, overlap=0, T=T, gamma=gamma, eps=eps, rope_dim=r,
                               rope_base=base), dtype, r)
    W = _store_like(O.compress(win_raw, None, None, None, m=1, overlap=0, T=i + 1, gamma=gamma, eps=eps,
                               rope_dim=r, rope_base=base, pos_stride=1), dtype, r)
    out = O.dense_mqa(q[None], E, W, q_pos=[i], m=m, n_win=n_win, eps=eps, sink=sink, rope_dim=r,
                      rope_base=base, scale=scale)[0]
    pre = O.pool_entries(Cf, Zf, None, None, m=m, overlap=0, T=T)
    pre[N - 1] = 1e3 * rng.standard_normal(c)        # stale newest entry: must not be read
    tb = m * (N - 1)
    p = dict(i=i, m=m, N=N, n_win=n_win, rope_dim=r, rope_base=base, eps=eps, scale=scale, dtype=dtype,
             C=Cf[tb:], Z=Zf[tb:], win_raw=win_raw[i - n_win + 1:], q=q, sink=sink)
    if with_gamma:
        p["gamma"] = gamma
    got = steps_mod.hca_decode_sequence(p, lambda s: pre[np.asarray(s)])
    np.testing.assert_allclose(got["out"], out, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype,k_dtype,with_gamma", [
    ("bf16", "e4m3", False), ("bf16", "bf16", False), ("f32", "f32", False), ("bf16", "mxfp4", False),
    ("mixed", "e4m3", True), ("bf16", "bf16", True)])
def test_csa_decode_step_equals_whole_sequence(dtype, k_dtype, with_gamma):
    from oracle import steps
    _csa_decode_pin(steps, dtype, k_dtype, with_gamma)


@pytest.mark.parametrize("dtype,with_gamma", [("bf16", False), ("f32", False), ("mixed", True)])
def test_hca_decode_step_equals_whole_sequence(dtype, with_gamma):
    from oracle import steps
    _hca_decode_pin(steps, dtype, with_gamma)


def _mutant_steps(old: str, new: str):
    """oracle.steps with one planted mistake (source text replaced once)."""
    import inspect
    import types

    from oracle import steps
    src = inspect.getsource(steps)
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle._steps_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<oracle.steps mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", [
    ("tok_base = m * (N - 2)", "tok_base = m * (N - 2) + 1"),          # block offset off by one
    ("tok_base = m * (N - 2)", "tok_base = m * (N - 2) - 1"),
    ("KI[N - 1] = k_new[0]", "KI[N - 2] = k_new[0]"),                   # wrong key row replaced
    ("rows[sel == N - 1] = e_new", "rows[sel == N - 2] = e_new"),       # wrong entry row replaced
    ("old = sel[sel != N - 1]", "old = sel[sel != -1]"),                # stale cache row read
    ("s_begin=N - 1, s_end=N, gamma=gam, eps=eps, rope_dim=r, rope_base=base)[0]\n    e_new = _store",
     "s_begin=N - 1, s_end=N, gamma=gam, eps=eps, rope_dim=r, rope_base=base, pos_offset=1)[0]\n"
     "    e_new = _store"),
    ("gam = p.get(\"gamma\")\n    e_new", "gam = None\n    e_new"),     # the norm weight dropped
    ("e_new = _store(e_new, p[\"dtype\"], r)", "e_new = _store(e_new, \"f64\", r)"),   # new entry unrounded
])
def test_csa_decode_pin_catches_planted_mistakes(old, new):
    bad = _mutant_steps(old, new)
    with pytest.raises((AssertionError, ValueError)):
        _csa_decode_pin(bad, "mixed", "e4m3", True)


@pytest.mark.parametrize("old,new", [
    ("tok_base=m * (N - 1),\n                       s_begin=N - 1",
     "tok_base=m * (N - 1) + 1,\n                       s_begin=N - 1"),   # block offset off by one
    ("E[N - 1] = _store(e_new", "E[N - 2] = _store(e_new"),              # wrong entry replaced
    ("E[: N - 1] = entry_rows(kv_raw_rows(s[: N - 1]), s[: N - 1]",
     "E[: N - 1] = entry_rows(kv_raw_rows(s[1: N]), s[: N - 1]"),         # rows shifted by one
    ("np.concatenate([E, W])", "np.concatenate([E, W[:-1]])"),        # window without the own token
    ("eps=eps, dtype=p[\"dtype\"], gamma=gam)\n    out = O.attend_one(p[\"q\"], np.concatenate([E, W])",
     "eps=eps, dtype=p[\"dtype\"])\n    out = O.attend_one(p[\"q\"], np.concatenate([E, W])"),   # window unweighted
])
def test_hca_decode_pin_catches_planted_mistakes(old, new):
    bad = _mutant_steps(old, new)
    with pytest.raises((AssertionError, ValueError)):
        _hca_decode_pin(bad, "mixed", True)


# ---------------------------------------------------------------------------
# MXFP4 (OCP MX v1.0: FP4 E2M1 elements, E8M0 scale per 32) for the FP4 indexer
# ---------------------------------------------------------------------------
def test_e2m1_codes_are_the_spec_table():
    """The 16 E2M1 codes: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0-7), the
    sign in bit 3 (OCP MX v1.0, FP4 E2M1 element format)."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oc.e2m1_to_f64(np.arange(16))
    assert list(got[:8]) == table
    assert list(-got[8:]) == table and np.all(np.signbit(got[8:]))
    assert [oc.e2m1_code(v) for v in table] == list(range(8))
    assert oc.e2m1_code(-0.0) == 8 and oc.e2m1_code(-6.0) == 15
    assert oc.e8m0_to_f64(127) == 1.0 and oc.e8m0_to_f64(0) == 2.0 ** -127
    assert oc.e8m0_to_f64(254) == 2.0 ** 127 and np.isnan(oc.e8m0_to_f64(255))


def _e2m1_brute(y: float) -> float:
    """Nearest E2M1 value by exhaustive search; ties to the even code (mantissa
    bit 0); beyond +-6 saturates."""
    mags = oc.e2m1_to_f64(np.arange(8))
    a = min(abs(y), 6.0)
    d = np.abs(mags - a)
    best = np.flatnonzero(d == d.min())
    code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
    return float(np.copysign(mags[code], y))


def test_e2m1_rne_matches_brute_force():
    rng = np.random.default_rng(31)
    mags = oc.e2m1_to_f64(np.arange(8))
    mids = (mags[1:] + mags[:-1]) / 2                      # every tie point
    ys = np.concatenate([rng.uniform(-9, 9, 4000), mids, -mids, mags, [6.5, 7.999, 100.0, -1e9, 0.25]])
    got = oc.f64_to_e2m1_value(ys)
    want = np.array([_e2m1_brute(y) for y in ys])
    assert np.array_equal(got, want)


def test_mx_shared_exponent_and_elements_brute_force():
    """Shared exponent = (largest e with 2^e <= block max) - 2, found by search over
    e; elements = E2M1 rounding of x / 2^shared; zero blocks take exponent -127."""
    rng = np.random.default_rng(32)
    rows = rng.standard_normal((40, 128)) * np.exp2(rng.integers(-30, 30, size=(40, 1)))
    rows[3, 32:64] = 0.0
    rows[5, :32] = np.exp2(rng.integers(-8, 8, size=32))   # powers of two exactly
    codes, sc = oc.mx_quantize_fp4(rows)
    for r in range(rows.shape[0]):
        for blk in range(4):
            x = rows[r, 32 * blk:32 * blk + 32]
            amax = np.max(np.abs(x))
            if amax == 0:
                assert sc[r, blk] == 0 and np.all(oc.e2m1_to_f64(codes[r, 32 * blk:32 * blk + 32]) == 0)
                continue
            e = max(e for e in range(-200, 200) if 2.0 ** e <= amax)
            assert sc[r, blk] == e - 2 + 127
            want = [_e2m1_brute(v / 2.0 ** (e - 2)) for v in x]
            assert np.array_equal(oc.e2m1_to_f64(codes[r, 32 * blk:32 * blk + 32]), want)


def test_mx_roundtrip_error_bound():
    """|x - dequant(quant(x))| is at most half the E2M1 spacing at |x| / X (times
    X), or |x| - 6 X for saturated elements, whose magnitude is below 8 X."""
    rng = np.random.default_rng(33)
    x = rng.standard_normal((64, 256)) * 3.7
    codes, sc = oc.mx_quantize_fp4(x)
    xh = oc.mx_fp4_to_f64(codes, sc)
    X = np.repeat(oc.e8m0_to_f64(sc), 32, axis=-1)
    y = np.abs(x) / X
    assert np.all(y < 8)
    spacing = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    bound = np.where(y <= 6, 0.5 * spacing * X, (y - 6) * X)
    assert np.all(np.abs(x - xh) <= bound * (1 + 1e-12))


def test_index_score_mxfp4_brute_force():
    """Tiny MXFP4 scores by plain loops over the decoded query and key values."""
    rng = np.random.default_rng(34)
    H, dI, N, m = 3, 64, 9, 2
    qI = oc.f64_to_bf16_value(rng.standard_normal((2, H, dI)))
    w = rng.standard_normal((2, H))
    Kc, Ks = oc.mx_quantize_fp4(rng.standard_normal((N, dI)) * 0.4)
    pos = [9, 17]
    got = O.index_score_mxfp4(qI, w, Kc, Ks, pos, m=m)
    for t in range(2):
        n_vis = min(N, (pos[t] + 1) // m)
        for s in range(N):
            if s >= n_vis:
                assert got[t, s] == -np.inf
                continue
            want = 0.0
            for h in range(H):
                qc, qs = oc.mx_quantize_fp4(qI[t, h])
                dot = 0.0
                for dd in range(dI):
                    qv = oc.e2m1_to_f64(qc[dd]) * 2.0 ** (int(qs[dd // 32]) - 127)
                    kv = oc.e2m1_to_f64(Kc[s, dd]) * 2.0 ** (int(Ks[s, dd // 32]) - 127)
                    dot += qv * kv
                want += w[t, h] * max(dot, 0.0)
            assert abs(got[t, s] - want) <= 1e-12 * max(1.0, abs(want))


def test_mx_planted_mistakes_are_caught(monkeypatch):
    # (1) shared exponent minus 1 instead of minus 2 (E2M1's emax taken as 1)
    with monkeypatch.context() as mp:
        mp.setattr(oc, "E2M1_EMAX", 1)
        with pytest.raises(AssertionError):
            test_mx_shared_exponent_and_elements_brute_force()
    # (2) ties rounded away from zero instead of to the even code
    real = oc.f64_to_e2m1_value

    def ties_away(x):
        x = np.asarray(x, dtype=np.float64)
        r = real(x)
        mags = oc.e2m1_to_f64(np.arange(8))
        mids = (mags[1:] + mags[:-1]) / 2
        up = {a: b for a, b in zip(mids, mags[1:])}
        return np.where(np.isin(np.abs(x), mids),
                        np.copysign([up.get(abs(v), 0.0) for v in x.ravel()], x.ravel()).reshape(x.shape), r)
    with monkeypatch.context() as mp:
        mp.setattr(oc, "f64_to_e2m1_value", ties_away)
        with pytest.raises(AssertionError):
            test_e2m1_rne_matches_brute_force()


# ---------------------------------------------------------------------------
# grouped output projection (method page §3.3)
# ---------------------------------------------------------------------------
def test_grouped_projection_equals_block_diagonal_matmul():
    """The grouped down-projection equals one product with a block-diagonal
    matrix built from the groups' matrices; g = 1 is two plain products."""
    from oracle.proj import grouped_output_projection as gop
    rng = np.random.default_rng(41)
    T, g, Wq, d_g, d = 5, 4, 6, 3, 7
    o = rng.standard_normal((T, g * Wq))
    W1 = rng.standard_normal((g, d_g, Wq))
    W2 = rng.standard_normal((d, g * d_g))
    y, out = gop(o, W1, W2, groups=g, y_dtype="f64")
    big = np.zeros((g * d_g, g * Wq))
    for q in range(g):
        big[q * d_g:(q + 1) * d_g, q * Wq:(q + 1) * Wq] = W1[q]
    np.testing.assert_allclose(y, o @ big.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out, (o @ big.T) @ W2.T, rtol=1e-12, atol=1e-12)
    # g = 1: two plain products
    W1one = rng.standard_normal((1, d_g, g * Wq))
    y1, out1 = gop(o, W1one, W2[:, :d_g], groups=1, y_dtype="f64")
    np.testing.assert_allclose(y1, o @ W1one[0].T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out1, (o @ W1one[0].T) @ W2[:, :d_g].T, rtol=1e-12, atol=1e-12)


def test_grouped_projection_brute_force_and_bf16_intermediate():
    from oracle.codecs import f64_to_bf16_value
    from oracle.proj import grouped_output_projection as gop
    rng = np.random.default_rng(42)
    T, g, Wq, d_g, d = 2, 3, 4, 2, 3
    o, W1, W2 = rng.standard_normal((T, g * Wq)), rng.standard_normal((g, d_g, Wq)), rng.standard_normal((d, g * d_g))
    y, out = gop(o, W1, W2, groups=g)
    for t in range(T):
        yb = []
        for q in range(g):
            for e in range(d_g):
                yb.append(sum(o[t, q * Wq + i] * W1[q, e, i] for i in range(Wq)))
        yb = f64_to_bf16_value(np.array(yb))
        assert np.array_equal(y[t], yb)
        for n in range(d):
            assert abs(out[t, n] - sum(yb[u] * W2[n, u] for u in range(g * d_g))) < 1e-12


def test_grouped_projection_planted_group_mixup_is_caught(monkeypatch):
    """A projection that gives group q the columns of group g-1-q fails the pins."""
    import oracle.proj as P
    real = P.grouped_output_projection

    def mixed(o, W1, W2, *, groups, y_dtype="bf16"):
        return real(o, W1[::-1].copy(), W2, groups=groups, y_dtype=y_dtype)
    with monkeypatch.context() as mp:
        mp.setattr(P, "grouped_output_projection", mixed)
        with pytest.raises(AssertionError):
            test_grouped_projection_equals_block_diagonal_matmul()


# ---------------------------------------------------------------------------
# heterogeneous cache maintenance (method page §3.5)
# ---------------------------------------------------------------------------
def _cache_tokens(rng, T, c=16, dI=8):
    tok = {k: rng.standard_normal((T, c)) for k in ("Ca", "Za", "Cb", "Zb", "Ch", "Zh", "Wraw")}
    tok.update({k: rng.standard_normal((T, dI)) for k in ("ICa", "IZa", "ICb", "IZb")})
    return tok


@pytest.mark.parametrize("chunks", [[1] * 70, [5, 1, 30, 2, 32], [70], [3, 64, 3]])
def test_incremental_cache_equals_full_recompression(chunks):
    """Appending tokens in any chunking, with only a ring of lcm(m, m') raw rows
    kept for the unfinished blocks, gives the caches that compressing the whole
    sequence gives (m = 4, m' = 16, so lcm = 16 and the ring wraps)."""
    from oracle import cache as Cc
    rng = np.random.default_rng(51)
    T = sum(chunks)
    m, m_hca, n_win, r = 4, 16, 6, 4
    tok = _cache_tokens(rng, T)
    kw = dict(m=m, m_hca=m_hca, n_win=n_win, rope_dim=r, rope_base=10000.0, eps=1e-6)
    R = Cc.ring_slots(m, m_hca)
    state = {"E_csa": [], "K_idx": [], "E_hca": [], "window": {}}
    ring = {k: np.full((R, tok[k].shape[1]), np.nan) for k in Cc.STREAMS_CSA + Cc.STREAMS_IDX + Cc.STREAMS_HCA}
    t0 = 0
    for n in chunks:
        t0 = Cc.append_incremental(state, ring, {k: v[t0:t0 + n] for k, v in tok.items()}, t0, **kw)
        full = Cc.cache_state(tok, t0, **kw)
        assert len(state["E_csa"]) == len(full["E_csa"]) == t0 // m
        assert len(state["E_hca"]) == len(full["E_hca"]) == t0 // m_hca
        if len(full["E_csa"]):
            np.testing.assert_allclose(np.stack(state["E_csa"]), full["E_csa"], rtol=0, atol=1e-12)
            np.testing.assert_allclose(np.stack(state["K_idx"]), full["K_idx"], rtol=0, atol=1e-12)
        if len(full["E_hca"]):
            np.testing.assert_allclose(np.stack(state["E_hca"]), full["E_hca"], rtol=0, atol=1e-12)
        assert sorted(state["window"]) == list(full["window_tokens"])
        np.testing.assert_allclose(np.stack([state["window"][t] for t in full["window_tokens"]]), full["window"],
                                   rtol=0, atol=1e-12)
        for k, rows in full["tail"].items():
            for u, t in enumerate(range(t0 - len(rows), t0)):
                assert np.array_equal(ring[k][t % R], rows[u])


def test_cache_ring_is_lcm_of_the_rates():
    from oracle import cache as Cc
    assert Cc.ring_slots(4, 16) == 16 and Cc.ring_slots(4, 128) == 128 and Cc.ring_slots(4, 6) == 12


def test_incremental_cache_planted_short_ring_is_caught():
    """A ring of m' - 1 slots loses the first token of an HCA block before the
    block completes: the pin fails."""
    from oracle import cache as Cc
    real = Cc.ring_slots
    Cc.ring_slots = lambda m, mh: real(m, mh) - 1
    try:
        with pytest.raises((AssertionError, ValueError)):
            test_incremental_cache_equals_full_recompression([1] * 70)
    finally:
        Cc.ring_slots = real


# ---------------------------------------------------------------------------
# mixed KV rows: RoPE dims bf16, the rest e4m3 with a row scale (method page §3.3)
# ---------------------------------------------------------------------------
def test_mixed_rows_split_into_the_two_codecs():
    """The mixed format is the e4m3 row quantisation of the first c - r channels
    and bf16 rounding of the last r, each checked against torch's own casts."""
    rng = np.random.default_rng(61)
    E = rng.standard_normal((20, 64)) * np.exp2(rng.integers(-4, 4, size=(20, 1)))
    r = 16
    vals, codes, sc = O.quantize_rows_mixed(E, r)
    x32 = torch.tensor(E[:, :48], dtype=torch.float32)
    amax = x32.abs().amax(dim=-1)
    want_sc = (amax / 448.0).numpy()
    assert np.array_equal(sc, want_sc)
    want_codes = (x32 / torch.tensor(want_sc)[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, want_codes)
    want_rope = torch.tensor(E[:, 48:]).to(torch.bfloat16).double().numpy()
    assert np.array_equal(vals[:, 48:], want_rope)
    assert np.all(np.abs(vals[:, :48] - E[:, :48]) <= 2.0 ** -4 * np.abs(E[:, :48]) + sc[:, None] * 2.0 ** -9)
