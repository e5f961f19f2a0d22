"""Device-resident steps of the CSA/HCA attention core, chained from the C-ABI calls.

Each class owns the device buffers of one workload (the compressed-entry
cache, the indexer-key cache, the sliding-window ring, the per-step inputs and
outputs) and runs one step in the order the DeepSeek-V4 method page (section
3.3) gives: compress what became complete, score with the lightning indexer,
select the top-k, attend (CSA) — or compress the tail block and attend densely
(HCA).  Everything runs in libcsa.so kernels on torch's current stream;
nothing here computes.

Cache set-up (untimed) stores N(0,1) "pre-norm" rows through csa_compress with
m = 1 (a single candidate, so pooling is the identity), which applies the
RMSNorm and the RoPE of each row's position exactly as for a freshly
compressed entry.
"""
from __future__ import annotations

import torch

from . import (CSA_E_UNSUPPORTED, CsaError, compress_jobs, csa_compress, csa_compress_batch,
               csa_compress_workspace_size,
               csa_decode_front, csa_index_score, csa_mqa_workspace_size, csa_sparse_mqa, csa_topk,
               csa_topk_workspace_size, hca_dense_mqa)

_TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _kv_rows(wl, rows: int, device):
    """A cache of KV rows (entries or window rows) in the workload's storage:
    (rows tensor, row scales or None).  Mixed rows are d + rope_dim bytes (e4m3
    codes of the first d - rope_dim dims, then the rotated dims as bf16) with
    one fp32 scale per row."""
    if wl.kv_dtype == "mixed":
        return (torch.zeros((wl.B, rows, wl.d + wl.rope_dim), dtype=torch.uint8, device=device),
                torch.zeros((wl.B, rows), dtype=torch.float32, device=device))
    return torch.zeros((wl.B, rows, wl.d), dtype=_TD[wl.kv_dtype], device=device), None


class _Common:
    E_scale = W_scale = None

    def _kv_gamma(self, g, wl):
        """RMSNorm weight of the entries and window rows: 1, or 1 + N(0, 1/16)."""
        from synth import workloads as W_
        if wl.kv_gamma == "normal":
            return (1.0 + 0.25 * g.normal(W_.T_GAMMA, (wl.d,), "f32", per_slot=False)).contiguous()
        return torch.ones(wl.d, dtype=torch.float32, device=self.dev)

    def _window_setup(self, g, wl, lo_tok: int, n_rows: int, tid_raw: int):
        """Window rows of tokens lo_tok .. lo_tok + n_rows - 1 into the ring W."""
        B, d = wl.B, wl.d
        self.win_raw = g.normal(tid_raw, (B, n_rows, d), wl.dtype)
        self.W, self.W_scale = _kv_rows(wl, wl.W_cap, self.dev)
        self._win_rows(lo_tok, lo_tok + n_rows, self.win_raw, lo_tok)

    def _win_job(self, s0: int, s1: int, raw: torch.Tensor, tok_base: int):
        """The window rows of tokens s0 .. s1 - 1 as a compression job (m = 1)."""
        wl = self.wl
        return (raw, None, None, None, self.W,
                dict(T=s1, m=1, overlap=0, s_begin=s0, s_end=s1, tok_base=tok_base, gamma=self.gamma_kv,
                     eps=wl.eps, rope_dim=wl.rope_dim, rope_base=wl.rope_base, pos_stride=1,
                     out_ring=wl.W_cap, E_scale=self.W_scale))

    def _win_rows(self, s0: int, s1: int, raw: torch.Tensor, tok_base: int):
        C_a, Z_a, C_b, Z_b, E, kw = self._win_job(s0, s1, raw, tok_base)
        csa_compress(C_a, Z_a, C_b, Z_b, E, **kw)

    def _fill_entries(self, E, raw, m: int, normalize: bool, rope: bool, E_scale=None):
        wl = self.wl
        N = raw.shape[1]
        csa_compress(raw, None, None, None, E, T=N, m=1, overlap=0, s_begin=0, s_end=N,
                     gamma=self.gamma_kv if normalize else None, eps=wl.eps,
                     rope_dim=wl.rope_dim if rope else 0, rope_base=wl.rope_base, pos_stride=m,
                     E_scale=E_scale)


class CSADecode(_Common):
    """CSA decode: one new query token per sequence at position q_pos0.

    Step: window row of the new token; recompress of the newest complete block
    (KV entry with norm + RoPE, indexer key without); indexer score over every
    visible entry; top-k; sparse MQA over the k entries + window + sink.
    """

    def __init__(self, wl, device="cuda", keep_raw: bool = True):
        from synth import Gen, workloads as W_
        self.wl, self.dev = wl, torch.device(device)
        g = Gen(wl.wid, self.dev)
        B, N, d, m, i = wl.B, wl.N_cap, wl.d, wl.m, wl.q_pos0
        assert wl.Tq == 1 and i >= m * N, "decode: every cached entry is complete"
        self.i = i
        self.gamma_kv = self._kv_gamma(g, wl)
        self.gamma_q = torch.ones(d, dtype=torch.float32, device=self.dev)
        # caches
        kv_raw = g.normal(W_.T_KVRAW, (B, N, d), wl.dtype)
        self.E, self.E_scale = _kv_rows(wl, N, self.dev)
        self._fill_entries(self.E, kv_raw, m, True, True, E_scale=self.E_scale)
        self.kv_raw = kv_raw if keep_raw else None
        self.KI_raw = None
        if wl.k_dtype == "e4m3":
            self.KI, self.KI_scale = g.normal_e4m3(W_.T_KI, (B, N, wl.d_I))
        elif wl.k_dtype == "mxfp4":
            # fp32 rows stored as MXFP4 by the compressor with m = 1 (pooling is the identity)
            raw = g.normal(W_.T_KI, (B, N, wl.d_I), "f32")
            self.KI = torch.empty((B, N, wl.d_I // 2), dtype=torch.uint8, device=self.dev)
            self.KI_scale = torch.empty((B, N, wl.d_I // 32), dtype=torch.uint8, device=self.dev)
            csa_compress(raw, None, None, None, self.KI, T=N, m=1, overlap=0, s_begin=0, s_end=N,
                         E_scale=self.KI_scale)
            self.KI_raw = raw if keep_raw else None
        else:
            self.KI, self.KI_scale = g.normal(W_.T_KI, (B, N, wl.d_I), wl.k_dtype), None
        self._window_setup(g, wl, i - wl.n_win + 1, wl.n_win, W_.T_WINRAW)
        self.win_new = self.win_raw[:, -1:].contiguous()
        # candidates of the newest complete block (entry N - 1) and the block before it
        self.blk_tok_base = m * (N - 2)
        R = 2 * m
        self.Ca, self.Za, self.Cb, self.Zb = (g.normal(t, (B, R, d), wl.dtype)
                                              for t in (W_.T_CA, W_.T_ZA, W_.T_CB, W_.T_ZB))
        self.ICa, self.IZa, self.ICb, self.IZb = (g.normal(t, (B, R, wl.d_I), wl.dtype)
                                                  for t in (W_.T_ICA, W_.T_IZA, W_.T_ICB, W_.T_IZB))
        # queries
        self.qI = g.normal(W_.T_QI, (B, 1, wl.H_I, wl.d_I), "bf16" if wl.k_dtype != "f32" else "f32")
        self.wI = g.uniform(W_.T_WI, (B, 1, wl.H_I))
        self.q = g.normal(W_.T_Q, (B, 1, wl.n_h, d), wl.dtype)
        self.sink = (g.normal(W_.T_SINK, (wl.n_h,), "f32", per_slot=False) if wl.sink == "normal"
                     else torch.zeros(wl.n_h, dtype=torch.float32, device=self.dev))
        self.q_pos = torch.full((B, 1), i, dtype=torch.int32, device=self.dev)
        # outputs and workspaces
        self.I = torch.empty((B, 1, N), dtype=torch.float32, device=self.dev)
        self.idx = torch.empty((B, 1, wl.k), dtype=torch.int32, device=self.dev)
        self.out = torch.empty_like(self.q)
        self.ws_topk = _ws(csa_topk_workspace_size(B, 1, N, wl.k), self.dev)
        self.ws_mqa = _ws(csa_mqa_workspace_size(B, 1, wl.n_h, d, wl.k + wl.n_win), self.dev)
        self.fused_front = None   # decided by the first front()
        self._jobs = None

    # -- the step ------------------------------------------------------------
    def _new_row_jobs(self):
        """The step's three compressions: the new token's window row, the newest
        KV entry and its indexer key (entry N - 1, the block just completed),
        marshalled once."""
        if self._jobs is None:
            self._jobs = compress_jobs(self._new_row_job_list())
        return self._jobs

    def _new_row_job_list(self):
        wl, i, N = self.wl, self.i, self.wl.N_cap
        T_done = wl.m * N
        return [
            self._win_job(i, i + 1, self.win_new, i),
            (self.Ca, self.Za, self.Cb, self.Zb, self.E,
             dict(T=T_done, m=wl.m, overlap=1, s_begin=N - 1, s_end=N, tok_base=self.blk_tok_base,
                  gamma=self.gamma_kv, eps=wl.eps, rope_dim=wl.rope_dim, rope_base=wl.rope_base,
                  E_scale=self.E_scale)),
            (self.ICa, self.IZa, self.ICb, self.IZb, self.KI,
             dict(T=T_done, m=wl.m, overlap=1, s_begin=N - 1, s_end=N, tok_base=self.blk_tok_base,
                  E_scale=self.KI_scale)),
        ]

    def compress_new(self):
        """The three compressions in one launch of their own."""
        csa_compress_batch(self._new_row_jobs())

    def front(self):
        """Compressions and indexer scores: one launch (csa_decode_front) where
        the library covers the combination (fp8 or bf16 keys, bf16 rows),
        otherwise the two launches.  ``fused_front`` records which ran."""
        if self.fused_front is not False:
            try:
                csa_decode_front(self._new_row_jobs(), self.qI, self.wI, self.KI, self.q_pos, self.I,
                                 m=self.wl.m, K_scale=self.KI_scale)
                self.fused_front = True
                return
            except CsaError as e:
                if e.status != CSA_E_UNSUPPORTED:
                    raise
                self.fused_front = False
        self.compress_new()
        self.index()

    def index(self):
        csa_index_score(self.qI, self.wI, self.KI, self.q_pos, self.I, m=self.wl.m, K_scale=self.KI_scale)

    def select(self):
        csa_topk(self.I, self.q_pos, self.idx, m=self.wl.m, k=self.wl.k, workspace=self.ws_topk)

    def attend(self):
        wl = self.wl
        csa_sparse_mqa(self.q, self.E, self.idx, self.W, self.q_pos, self.out, n_win=wl.n_win,
                       sink=self.sink, gamma_q=self.gamma_q, eps=wl.eps, rope_dim=wl.rope_dim,
                       rope_base=wl.rope_base, scale=wl.scale, workspace=self.ws_mqa,
                       E_scale=self.E_scale, W_scale=self.W_scale)

    def step(self):
        self.front()
        self.select()
        self.attend()

    # -- accounting -----------------------------------------------------------
    def algorithmic_bytes(self) -> dict:
        """Bytes every step must move at least once (inputs read, outputs written)."""
        wl = self.wl
        B, N, d, dI, H, k = wl.B, wl.N_cap, wl.d, wl.d_I, wl.H_I, wl.k
        esz = {"e4m3": 1, "bf16": 2, "f32": 4}
        kv = esz[wl.dtype]
        keys = B * N * dI * esz[wl.k_dtype] + (B * N * 4 if wl.k_dtype == "e4m3" else 0)
        index_io = B * (H * dI * 2 + H * 4)
        scores = B * N * 4
        gather = B * k * d * kv
        window = B * wl.n_win * d * kv
        qo = 2 * B * wl.n_h * d * kv
        # candidates of the newest block pair, the new window row (read + write), the new
        # KV entry and the new indexer key (+ its scale)
        compress = B * (4 * 2 * wl.m * (d + dI) * kv + 3 * d * kv + dI * esz[wl.k_dtype] + 4)
        idx = 2 * B * k * 4
        return {"index_kernel": keys + index_io + scores,
                "step": keys + index_io + gather + window + qo + compress + idx,
                "keys": keys, "gather": gather}

    def index_flops(self) -> float:
        wl = self.wl
        return 2.0 * wl.B * wl.N_cap * wl.H_I * wl.d_I


class HCADecode(_Common):
    """HCA decode: recompress the just-completed 128-token block, then dense MQA
    over every visible entry plus window and sink."""

    def __init__(self, wl, device="cuda", keep_raw: bool = True):
        from synth import Gen, workloads as W_
        self.wl, self.dev = wl, torch.device(device)
        g = Gen(wl.wid, self.dev)
        B, N, d, m, i = wl.B, wl.N_cap, wl.d, wl.m, wl.q_pos0
        self.i = i
        self.gamma_kv = self._kv_gamma(g, wl)
        self.gamma_q = torch.ones(d, dtype=torch.float32, device=self.dev)
        kv_raw = g.normal(W_.T_KVRAW, (B, N, d), wl.dtype)
        self.E, self.E_scale = _kv_rows(wl, N, self.dev)
        self._fill_entries(self.E, kv_raw, m, True, True, E_scale=self.E_scale)
        self.kv_raw = kv_raw if keep_raw else None
        self._window_setup(g, wl, i - wl.n_win + 1, wl.n_win, W_.T_WINRAW)
        self.win_new = self.win_raw[:, -1:].contiguous()
        self.blk_tok_base = m * (N - 1)
        self.C = g.normal(W_.T_CA, (B, m, d), wl.dtype)
        self.Z = g.normal(W_.T_ZA, (B, m, d), wl.dtype)
        self.q = g.normal(W_.T_Q, (B, 1, wl.n_h, d), wl.dtype)
        self.sink = g.normal(W_.T_SINK, (wl.n_h,), "f32", per_slot=False)
        self.q_pos = torch.full((B, 1), i, dtype=torch.int32, device=self.dev)
        self.out = torch.empty_like(self.q)
        self.ws_mqa = _ws(csa_mqa_workspace_size(B, 1, wl.n_h, d, N + wl.n_win), self.dev)
        # the compressor's channel-split workspace (pooled rows between its two kernels)
        self.ws_compress = _ws(csa_compress_workspace_size(self._compress_jobs()), self.dev)

    def _compress_jobs(self):
        wl, i, N = self.wl, self.i, self.wl.N_cap
        return [
            self._win_job(i, i + 1, self.win_new, i),
            (self.C, self.Z, None, None, self.E,
             dict(T=wl.m * N, m=wl.m, overlap=0, s_begin=N - 1, s_end=N, tok_base=self.blk_tok_base,
                  gamma=self.gamma_kv, eps=wl.eps, rope_dim=wl.rope_dim, rope_base=wl.rope_base,
                  E_scale=self.E_scale)),
        ]

    def compress_new(self):
        """The new token's window row and the just-completed block's entry, one
        launch (the entry's 512 channels pooled by 8 workgroups)."""
        csa_compress_batch(self._compress_jobs(), workspace=self.ws_compress)

    def attend(self):
        wl = self.wl
        hca_dense_mqa(self.q, self.E, self.W, self.q_pos, self.out, m=wl.m, n_win=wl.n_win,
                      sink=self.sink, gamma_q=self.gamma_q, eps=wl.eps, rope_dim=wl.rope_dim,
                      rope_base=wl.rope_base, scale=wl.scale, workspace=self.ws_mqa,
                      E_scale=self.E_scale, W_scale=self.W_scale)

    def step(self):
        self.compress_new()
        self.attend()


class CSAPrefill(_Common):
    """CSA chunked prefill: Tq queries at positions q_pos0 .. q_pos0 + Tq - 1.

    Step: window rows of the chunk's tokens; compression of the entries that
    complete inside the chunk (KV entries and indexer keys); indexer scores of
    every query; top-k per query; sparse MQA."""

    def __init__(self, wl, device="cuda", keep_raw: bool = True):
        from synth import Gen, workloads as W_
        self.wl, self.dev = wl, torch.device(device)
        g = Gen(wl.wid, self.dev)
        B, N, d, m, Tq, p0 = wl.B, wl.N_cap, wl.d, wl.m, wl.Tq, wl.q_pos0
        self.gamma_kv = self._kv_gamma(g, wl)
        self.gamma_q = torch.ones(d, dtype=torch.float32, device=self.dev)
        # entries completed before the chunk come from the cache; those inside it are compressed
        self.s_new0, self.s_new1 = p0 // m, (p0 + Tq) // m
        kv_raw = g.normal(W_.T_KVRAW, (B, N, d), wl.dtype)
        self.E = torch.empty((B, N, d), dtype=_TD[wl.dtype], device=self.dev)
        self._fill_entries(self.E, kv_raw, m, True, True)
        self.kv_raw = kv_raw if keep_raw else None
        self.KI = g.normal(W_.T_KI, (B, N, wl.d_I), wl.k_dtype)
        self.KI_init = self.KI.clone() if keep_raw else None   # the cache before the step
        # window ring: the 127 tokens before the chunk from set-up, the chunk's own rows per step
        self._window_setup(g, wl, p0 - (wl.n_win - 1), wl.n_win - 1, W_.T_WINRAW)
        self.chunk_raw = g.normal(W_.T_WINRAW + 100, (B, Tq, d), wl.dtype)
        # candidates of the chunk (plus the block before it, for the overlapping set b)
        self.tok_base = m * (self.s_new0 - 1)
        R = p0 + Tq - self.tok_base
        self.Ca, self.Za, self.Cb, self.Zb = (g.normal(t, (B, R, d), wl.dtype)
                                              for t in (W_.T_CA, W_.T_ZA, W_.T_CB, W_.T_ZB))
        self.ICa, self.IZa, self.ICb, self.IZb = (g.normal(t, (B, R, wl.d_I), wl.dtype)
                                                  for t in (W_.T_ICA, W_.T_IZA, W_.T_ICB, W_.T_IZB))
        self.qI = g.normal(W_.T_QI, (B, Tq, wl.H_I, wl.d_I), "bf16")
        self.wI = g.uniform(W_.T_WI, (B, Tq, wl.H_I))
        self.q = g.normal(W_.T_Q, (B, Tq, wl.n_h, d), wl.dtype)
        self.sink = g.normal(W_.T_SINK, (wl.n_h,), "f32", per_slot=False)
        self.q_pos = (p0 + torch.arange(Tq, dtype=torch.int32, device=self.dev)).repeat(B, 1).contiguous()
        self.I = torch.empty((B, Tq, N), dtype=torch.float32, device=self.dev)
        self.idx = torch.empty((B, Tq, wl.k), dtype=torch.int32, device=self.dev)
        self.out = torch.empty_like(self.q)
        self.ws_topk = _ws(csa_topk_workspace_size(B, Tq, N, wl.k), self.dev)
        self.ws_mqa = _ws(csa_mqa_workspace_size(B, Tq, wl.n_h, d, wl.k + wl.n_win), self.dev)

    def compress_new(self):
        """The chunk's window rows, its complete KV entries and their indexer
        keys: three independent compressions, one launch."""
        wl = self.wl
        p0, Tq = wl.q_pos0, wl.Tq
        T = p0 + Tq
        csa_compress_batch([
            self._win_job(p0, p0 + Tq, self.chunk_raw, p0),
            (self.Ca, self.Za, self.Cb, self.Zb, self.E,
             dict(T=T, m=wl.m, overlap=1, s_begin=self.s_new0, s_end=self.s_new1, tok_base=self.tok_base,
                  gamma=self.gamma_kv, eps=wl.eps, rope_dim=wl.rope_dim, rope_base=wl.rope_base)),
            (self.ICa, self.IZa, self.ICb, self.IZb, self.KI,
             dict(T=T, m=wl.m, overlap=1, s_begin=self.s_new0, s_end=self.s_new1, tok_base=self.tok_base)),
        ])

    def index(self):
        csa_index_score(self.qI, self.wI, self.KI, self.q_pos, self.I, m=self.wl.m)

    def select(self):
        csa_topk(self.I, self.q_pos, self.idx, m=self.wl.m, k=self.wl.k, workspace=self.ws_topk)

    def attend(self):
        wl = self.wl
        csa_sparse_mqa(self.q, self.E, self.idx, self.W, self.q_pos, self.out, n_win=wl.n_win,
                       sink=self.sink, gamma_q=self.gamma_q, eps=wl.eps, rope_dim=wl.rope_dim,
                       rope_base=wl.rope_base, scale=wl.scale, workspace=self.ws_mqa)

    def step(self):
        self.compress_new()
        self.index()
        self.select()
        self.attend()

    def causal_index_flops(self) -> float:
        """2 * H_I * d_I flops per visible (query, entry) pair."""
        wl = self.wl
        pairs = sum(min(wl.N_cap, (wl.q_pos0 + t + 1) // wl.m) for t in range(wl.Tq))
        return 2.0 * wl.B * pairs * wl.H_I * wl.d_I
