"""CSA/HCA hybrid-attention core for AMD Instinct MI355X (gfx950).

A thin binding over ``libcsa.so`` (hand-written HIP kernels behind the C ABI
of ``include/csa.h``).  Functions carry the C names and only marshal
arguments: tensors become device pointers, their shapes fill the size
arguments, and work is enqueued on torch's current HIP stream.  Every step of
the computation runs in the library's kernels; there is no fallback: if the
library is missing, importing this package raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "CsaError", "LIB_PATH", "abi_version", "csa_compress", "csa_compress_batch", "csa_compress_workspace_size",
    "CompressJobs", "compress_jobs",
    "csa_index_score", "csa_decode_front", "CSA_E_UNSUPPORTED",
    "csa_topk",
    "csa_topk_workspace_size", "csa_sparse_mqa", "csa_sparse_mqa_noalloc", "hca_dense_mqa",
    "csa_mqa_workspace_size", "NOALLOC_SCRATCH_BYTES", "csa_out_proj_workspace_size",
    "csa_grouped_out_proj", "csa_cache_append", "cache_ring_slots",
    "CSA_F32", "CSA_BF16", "CSA_FP8_E4M3", "CSA_MXFP4", "CSA_KV_MIXED",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
CSA_F32, CSA_BF16, CSA_FP8_E4M3, CSA_MXFP4, CSA_KV_MIXED = 0, 1, 2, 3, 4
CSA_E_UNSUPPORTED = 4

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python long_context_attention_02_amd/build.py` "
        "(or __graft_entry__.build()); the CSA/HCA core has no non-HIP implementation")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_longlong
_F = ctypes.c_float
_S = ctypes.c_size_t

_lib.csa_abi_version.restype = _I
_lib.csa_status_str.restype = ctypes.c_char_p
_lib.csa_status_str.argtypes = [_I]
_lib.csa_last_error.restype = ctypes.c_char_p
_lib.csa_compress.restype = _I
_lib.csa_compress.argtypes = [_P, _P, _P, _P, _I, _I, _L, _L, _L, _L, _P, _I, _I, _I, _L, _L, _P, _F,
                              _I, _F, _L, _L, _P, _I, _P, _L, _L, _P]


class _CompressJob(ctypes.Structure):
    """csa_compress_job of include/csa.h (C layout, natural alignment)."""
    _fields_ = [("C_a", _P), ("Z_a", _P), ("C_b", _P), ("Z_b", _P), ("in_dtype", _I), ("B", _I),
                ("R", _L), ("in_batch_stride", _L), ("tok_base", _L), ("T", _L), ("T_len", _P),
                ("c", _I), ("m", _I), ("overlap", _I), ("s_begin", _L), ("s_end", _L),
                ("gamma", _P), ("eps", _F), ("rope_dim", _I), ("rope_base", _F),
                ("pos_stride", _L), ("pos_offset", _L), ("E", _P), ("out_dtype", _I),
                ("E_scale", _P), ("out_batch_stride", _L), ("out_ring", _L)]


_lib.csa_compress_batch.restype = _I
_lib.csa_compress_batch.argtypes = [ctypes.POINTER(_CompressJob), _I, _P, _S, _P]
_lib.csa_compress_workspace_size.restype = _S
_lib.csa_compress_workspace_size.argtypes = [ctypes.POINTER(_CompressJob), _I]
_lib.csa_index_score.restype = _I
_lib.csa_index_score.argtypes = [_P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _I, _L, _I, _P, _P]
_lib.csa_decode_front.restype = _I
_lib.csa_decode_front.argtypes = [ctypes.c_void_p, _I, _P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _L, _I, _P, _P]
_lib.csa_topk_workspace_size.restype = _S
_lib.csa_topk_workspace_size.argtypes = [_I, _I, _L, _I]
_lib.csa_topk.restype = _I
_lib.csa_topk.argtypes = [_P, _P, _I, _I, _L, _I, _I, _P, _P, _P, _S, _P]
_lib.csa_mqa_workspace_size.restype = _S
_lib.csa_mqa_workspace_size.argtypes = [_I, _I, _I, _I, _L]
_lib.csa_sparse_mqa.restype = _I
_lib.csa_sparse_mqa.argtypes = [_P, _P, _F, _P, _P, _L, _P, _I, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I,
                                _I, _F, _F, _I, _P, _P, _S, _P]
_lib.csa_sparse_mqa_noalloc.restype = _I
_lib.csa_sparse_mqa_noalloc.argtypes = [_P, _P, _F, _P, _P, _L, _P, _I, _P, _P, _I, _I, _P, _P, _I, _I,
                                        _I, _I, _I, _F, _F, _I, _P, _P]
NOALLOC_SCRATCH_BYTES = 16 << 20
_lib.csa_cache_append.restype = _I
_lib.csa_cache_append.argtypes = [_I, _P, _I, _I, _I, _I, _I] + [_P] * 15 + [_I, _L, _P, _L, _P, _I, _P, _F, _I,
                                                                              _F, _P]
_lib.csa_out_proj_workspace_size.restype = _S
_lib.csa_out_proj_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
_lib.csa_grouped_out_proj.restype = _I
_lib.csa_grouped_out_proj.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _S, _P]
_lib.hca_dense_mqa.restype = _I
_lib.hca_dense_mqa.argtypes = [_P, _P, _F, _P, _P, _L, _I, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I,
                               _I, _F, _F, _I, _P, _P, _S, _P]


class CsaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        name = _lib.csa_status_str(status).decode()
        super().__init__(f"{name} ({status}): {detail}")


def abi_version() -> int:
    return _lib.csa_abi_version()


def _check(status: int):
    if status != 0:
        raise CsaError(status, _lib.csa_last_error().decode())


# uint8 tensors hold MXFP4 (two E2M1 codes per byte, E8M0 block scales beside them)
_DT = {torch.float32: CSA_F32, torch.bfloat16: CSA_BF16, torch.float8_e4m3fn: CSA_FP8_E4M3,
       torch.uint8: CSA_MXFP4}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t, name, dtype=None, dims=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _compress_args(C_a, Z_a, C_b, Z_b, E, *, T: int, m: int, overlap: int, s_begin: int,
                   s_end: int, tok_base: int = 0, gamma=None, eps: float = 1e-6, rope_dim: int = 0,
                   rope_base: float = 10000.0, pos_stride: int | None = None, pos_offset: int = 0,
                   E_scale=None, out_ring: int = 0, T_len=None):
    """The C arguments of one compression (without the stream), in csa_compress order."""
    B, R, c = C_a.shape
    for name, t in (("Z_a", Z_a), ("C_b", C_b), ("Z_b", Z_b)):
        if t is not None and (t.shape != C_a.shape or t.dtype != C_a.dtype):
            raise ValueError(f"{name} must match C_a in shape and dtype")
    # uint8 rows: mixed (c + rope_dim bytes: fp8 codes, then bf16 rotated dims) or MXFP4 (c / 2)
    mixed = E.dtype == torch.uint8 and E.dim() == 3 and rope_dim > 0 and E.shape[2] == c + rope_dim
    mx = E.dtype == torch.uint8 and not mixed
    if E.dim() != 3 or E.shape[0] != B or E.shape[2] != (c // 2 if mx else c + rope_dim if mixed else c):
        raise ValueError("E must be [B, rows, c] ([B, rows, c / 2] bytes for MXFP4, "
                         "[B, rows, c + rope_dim] for mixed rows)")
    if E.shape[1] < (out_ring if out_ring > 0 else s_end):
        raise ValueError("E has fewer rows than the entries written")
    if mx and (E_scale is None or E_scale.dtype != torch.uint8 or tuple(E_scale.shape) != (B, E.shape[1], c // 32)):
        raise ValueError("MXFP4 output needs E_scale uint8 [B, rows, c / 32]")
    if not mx and E_scale is not None and tuple(E_scale.shape) != (B, E.shape[1]):
        raise ValueError("E_scale must be [B, rows]")
    if T_len is not None and tuple(T_len.shape) != (B,):
        raise ValueError("T_len must be [B]")
    return (_ptr(C_a, "C_a", dims=3), _ptr(Z_a, "Z_a"), _ptr(C_b, "C_b"), _ptr(Z_b, "Z_b"), _dt(C_a),
            B, R, R * c, tok_base, T, _ptr(T_len, "T_len", torch.int32), c, m, overlap, s_begin, s_end,
            _ptr(gamma, "gamma", torch.float32), eps, rope_dim, rope_base,
            m if pos_stride is None else pos_stride, pos_offset,
            _ptr(E, "E"), CSA_KV_MIXED if mixed else _dt(E),
            _ptr(E_scale, "E_scale", torch.uint8 if mx else torch.float32), E.shape[1] * c, out_ring)


def csa_compress(C_a, Z_a, C_b, Z_b, E, **kw):
    """a1.  C_a/Z_a/C_b/Z_b: [B, R, c] (Z may be None; C_b None when overlap=0),
    E: [B, rows, c] float32 / bfloat16 / float8_e4m3fn, E_scale: [B, rows] fp32
    for fp8 output.  Row r of the candidates is token tok_base + r.  Keywords:
    T, m, overlap, s_begin, s_end (required); tok_base, gamma, eps, rope_dim,
    rope_base, pos_stride (default m), pos_offset, E_scale, out_ring, T_len ([B] int32
    per-sequence token counts, each <= T)."""
    _check(_lib.csa_compress(*_compress_args(C_a, Z_a, C_b, Z_b, E, **kw), _stream()))


class CompressJobs:
    """Job descriptors marshalled once (compress_jobs), for calls repeated on the
    same tensors: csa_compress_batch and csa_decode_front take it in place of
    the list.  It keeps the tensors alive."""

    def __init__(self, jobs):
        self.jobs = list(jobs)
        self.arr = (_CompressJob * max(len(self.jobs), 1))()
        for q, (C_a, Z_a, C_b, Z_b, E, kw) in enumerate(self.jobs):
            self.arr[q] = _CompressJob(*_compress_args(C_a, Z_a, C_b, Z_b, E, **kw))

    def __len__(self):
        return len(self.jobs)


def compress_jobs(jobs) -> CompressJobs:
    return jobs if isinstance(jobs, CompressJobs) else CompressJobs(jobs)


def _compress_jobs(jobs):
    return compress_jobs(jobs).arr


def csa_compress_workspace_size(jobs) -> int:
    """Bytes of the workspace csa_compress_batch takes for these jobs (0: none)."""
    return int(_lib.csa_compress_workspace_size(_compress_jobs(jobs), len(jobs)))


def csa_compress_batch(jobs, workspace=None):
    """a1, several compressions in one launch.  ``jobs`` is a list of
    (C_a, Z_a, C_b, Z_b, E, kwargs) with the arguments of csa_compress.
    Without a workspace the outputs equal those of the separate calls; with one
    (uint8 device tensor of csa_compress_workspace_size bytes) entries of many
    candidates pool their channels over several workgroups."""
    arr = _compress_jobs(jobs)
    wp, wb = (workspace.data_ptr(), workspace.numel() * workspace.element_size()) if workspace is not None \
        else (None, 0)
    _check(_lib.csa_compress_batch(arr, len(jobs), wp, wb, _stream()))


def csa_index_score(q_I, w_I, K_I, q_pos, I_out, *, m: int, K_scale=None):
    """a2.  q_I [B, Tq, H, dI], w_I [B, Tq, H] fp32, K_I [B, N, dI],
    q_pos [B, Tq] int32, I_out [B, Tq, N] fp32, K_scale [B, N] for fp8 keys.
    MXFP4 keys: K_I uint8 [B, N, dI / 2] and K_scale uint8 [B, N, dI / 32]."""
    B, Tq, H, dI = q_I.shape
    N = K_I.shape[1]
    mx = K_I.dtype == torch.uint8
    if tuple(w_I.shape) != (B, Tq, H) or K_I.shape[0] != B or K_I.shape[2] != (dI // 2 if mx else dI):
        raise ValueError("shape mismatch among q_I, w_I, K_I")
    if mx and (K_scale is None or K_scale.dtype != torch.uint8 or tuple(K_scale.shape) != (B, N, dI // 32)):
        raise ValueError("MXFP4 keys need K_scale uint8 [B, N, dI / 32]")
    if not mx and K_scale is not None and tuple(K_scale.shape) != (B, N):
        raise ValueError("K_scale must be [B, N]")
    if tuple(I_out.shape) != (B, Tq, N) or tuple(q_pos.shape) != (B, Tq):
        raise ValueError("I_out must be [B, Tq, N] and q_pos [B, Tq]")
    _check(_lib.csa_index_score(
        _ptr(q_I, "q_I", dims=4), _dt(q_I), _ptr(w_I, "w_I", torch.float32), _ptr(K_I, "K_I", dims=3),
        _dt(K_I), _ptr(K_scale, "K_scale", torch.uint8 if mx else torch.float32),
        _ptr(q_pos, "q_pos", torch.int32),
        B, Tq, H, dI, N, m, _ptr(I_out, "I_out", torch.float32), _stream()))


def csa_decode_front(jobs, q_I, w_I, K_I, q_pos, I_out, *, m: int, K_scale=None):
    """a1 + a2 of a decode step in one launch: the compressions ``jobs`` (as in
    csa_compress_batch; one of them writes K_I's last rows) beside the scores of
    csa_index_score (one query row per sequence: q_I [B, 1, H, dI], w_I [B, 1, H],
    q_pos [B, 1], I_out [B, 1, N]).  Raises CsaError with status
    CSA_E_UNSUPPORTED, having launched nothing, when the combination is not
    covered; the caller then makes the two separate calls."""
    B, Tq, H, dI = q_I.shape
    N = K_I.shape[1]
    if Tq != 1 or tuple(w_I.shape) != (B, 1, H) or tuple(q_pos.shape) != (B, 1) or tuple(I_out.shape) != (B, 1, N):
        raise ValueError("csa_decode_front: one query row per sequence (q_I [B, 1, H, dI], w_I [B, 1, H], "
                         "q_pos [B, 1], I_out [B, 1, N])")
    mx = K_I.dtype == torch.uint8
    if K_I.dim() != 3 or K_I.shape[0] != B or K_I.shape[2] != (dI // 2 if mx else dI):
        raise ValueError("K_I must be [B, N, dI] ([B, N, dI / 2] bytes for MXFP4)")
    if K_scale is not None and tuple(K_scale.shape) != ((B, N, dI // 32) if mx else (B, N)):
        raise ValueError("K_scale must be [B, N] ([B, N, dI / 32] bytes for MXFP4)")
    arr = _compress_jobs(jobs)
    _check(_lib.csa_decode_front(
        ctypes.cast(arr, ctypes.c_void_p), len(jobs), _ptr(q_I, "q_I", dims=4), _dt(q_I),
        _ptr(w_I, "w_I", torch.float32), _ptr(K_I, "K_I", dims=3), _dt(K_I),
        _ptr(K_scale, "K_scale", torch.uint8 if mx else torch.float32), _ptr(q_pos, "q_pos", torch.int32),
        B, H, dI, N, m, _ptr(I_out, "I_out", torch.float32), _stream()))


def csa_topk_workspace_size(B: int, Tq: int, N: int, k: int) -> int:
    return int(_lib.csa_topk_workspace_size(B, Tq, N, k))


def csa_topk(I, q_pos, idx_out, *, m: int, k: int, val_out=None, workspace=None):
    """a3.  I [B, Tq, N] fp32, idx_out [B, Tq, k] int32, val_out optional."""
    B, Tq, N = I.shape
    if tuple(idx_out.shape) != (B, Tq, k):
        raise ValueError("idx_out must be [B, Tq, k]")
    if val_out is not None and tuple(val_out.shape) != (B, Tq, k):
        raise ValueError("val_out must be [B, Tq, k]")
    if tuple(q_pos.shape) != (B, Tq):
        raise ValueError("q_pos must be [B, Tq]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.csa_topk(
        _ptr(I, "I", torch.float32, 3), _ptr(q_pos, "q_pos", torch.int32), B, Tq, N, m, k,
        _ptr(idx_out, "idx_out", torch.int32), _ptr(val_out, "val_out", torch.float32),
        _ptr(workspace, "workspace"), ws_bytes, _stream()))


def csa_mqa_workspace_size(B: int, Tq: int, n_h: int, d: int, n_keys_max: int) -> int:
    return int(_lib.csa_mqa_workspace_size(B, Tq, n_h, d, n_keys_max))


def _mqa_common(q, E, W, q_pos, out, sink, gamma_q, rope_dim=0, E_scale=None, W_scale=None):
    """Shape checks; returns (B, Tq, n_h, d, dtype code, E_scale ptr, W_scale ptr).  uint8 E and W
    are mixed rows of d + rope_dim bytes with fp32 row scales E_scale [B, N], W_scale [B, W_cap]."""
    B, Tq, n_h, d = q.shape
    mixed = E.dtype == torch.uint8
    row = d + rope_dim if mixed else d
    kv_dt = torch.uint8 if mixed else q.dtype
    if mixed and q.dtype != torch.bfloat16:
        raise TypeError("mixed entries need bf16 queries")
    if E.dim() != 3 or E.shape[0] != B or E.shape[2] != row or E.dtype != kv_dt:
        raise ValueError("E must be [B, N, d] with q's dtype (uint8 [B, N, d + rope_dim] mixed rows)")
    if W is not None and (W.dim() != 3 or W.shape[0] != B or W.shape[2] != row or W.dtype != kv_dt):
        raise ValueError("W must be laid out as E ([B, W_cap, ...])")
    es = ws = None
    if mixed:
        if E_scale is None or tuple(E_scale.shape) != (B, E.shape[1]):
            raise ValueError("mixed entries need E_scale [B, N]")
        es = _ptr(E_scale, "E_scale", torch.float32)
        if W is not None:
            if W_scale is None or tuple(W_scale.shape) != (B, W.shape[1]):
                raise ValueError("mixed window rows need W_scale [B, W_cap]")
            ws = _ptr(W_scale, "W_scale", torch.float32)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(q_pos.shape) != (B, Tq):
        raise ValueError("q_pos must be [B, Tq]")
    if sink is not None and tuple(sink.shape) != (n_h,):
        raise ValueError("sink must be [n_h]")
    if gamma_q is not None and tuple(gamma_q.shape) != (d,):
        raise ValueError("gamma_q must be [d]")
    return B, Tq, n_h, d, (CSA_KV_MIXED if mixed else _dt(q)), es, ws


def csa_sparse_mqa(q, E, idx, W, q_pos, out, *, n_win: int, sink=None, gamma_q=None, eps: float = 1e-6,
                   rope_dim: int = 0, rope_base: float = 10000.0, scale: float | None = None,
                   workspace=None, E_scale=None, W_scale=None):
    """a4.  q [B, Tq, n_h, d], E [B, N, d], idx [B, Tq, k] int32, W [B, W_cap, d]
    or None, q_pos [B, Tq] int32, out like q; sink [n_h], gamma_q [d] fp32.
    Mixed entries: E uint8 [B, N, d + rope_dim] with E_scale [B, N] fp32, W
    likewise with W_scale [B, W_cap]; q and out bf16."""
    B, Tq, n_h, d, dt, es, wsc = _mqa_common(q, E, W, q_pos, out, sink, gamma_q, rope_dim, E_scale, W_scale)
    k = idx.shape[2]
    if tuple(idx.shape[:2]) != (B, Tq):
        raise ValueError("idx must be [B, Tq, k]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.csa_sparse_mqa(
        _ptr(q, "q", dims=4), _ptr(gamma_q, "gamma_q", torch.float32), eps, _ptr(E, "E"), es, E.shape[1],
        _ptr(idx, "idx", torch.int32, 3), k, _ptr(W, "W"), wsc, 0 if W is None else W.shape[1], n_win,
        _ptr(sink, "sink", torch.float32), _ptr(q_pos, "q_pos", torch.int32), B, Tq, n_h, d,
        rope_dim, rope_base, (d ** -0.5) if scale is None else scale, dt, _ptr(out, "out"),
        _ptr(workspace, "workspace"), ws_bytes, _stream()))


def csa_sparse_mqa_noalloc(q, E, idx, W, q_pos, out, *, n_win: int, sink=None, gamma_q=None,
                           eps: float = 1e-6, rope_dim: int = 0, rope_base: float = 10000.0,
                           scale: float | None = None, E_scale=None, W_scale=None):
    """a4 without a workspace: the split partials live in the library's static
    per-GPU scratch (NOALLOC_SCRATCH_BYTES); calls that overlap on one GPU race."""
    B, Tq, n_h, d, dt, es, wsc = _mqa_common(q, E, W, q_pos, out, sink, gamma_q, rope_dim, E_scale, W_scale)
    k = idx.shape[2]
    if tuple(idx.shape[:2]) != (B, Tq):
        raise ValueError("idx must be [B, Tq, k]")
    _check(_lib.csa_sparse_mqa_noalloc(
        _ptr(q, "q", dims=4), _ptr(gamma_q, "gamma_q", torch.float32), eps, _ptr(E, "E"), es, E.shape[1],
        _ptr(idx, "idx", torch.int32, 3), k, _ptr(W, "W"), wsc, 0 if W is None else W.shape[1], n_win,
        _ptr(sink, "sink", torch.float32), _ptr(q_pos, "q_pos", torch.int32), B, Tq, n_h, d,
        rope_dim, rope_base, (d ** -0.5) if scale is None else scale, dt, _ptr(out, "out"),
        _stream()))


def hca_dense_mqa(q, E, W, q_pos, out, *, m: int, n_win: int, sink=None, gamma_q=None, eps: float = 1e-6,
                  rope_dim: int = 0, rope_base: float = 10000.0, scale: float | None = None,
                  workspace=None, E_scale=None, W_scale=None):
    """a5.  As csa_sparse_mqa over every visible entry s < floor((i+1)/m)."""
    B, Tq, n_h, d, dt, es, wsc = _mqa_common(q, E, W, q_pos, out, sink, gamma_q, rope_dim, E_scale, W_scale)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.hca_dense_mqa(
        _ptr(q, "q", dims=4), _ptr(gamma_q, "gamma_q", torch.float32), eps, _ptr(E, "E"), es, E.shape[1], m,
        _ptr(W, "W"), wsc, 0 if W is None else W.shape[1], n_win, _ptr(sink, "sink", torch.float32),
        _ptr(q_pos, "q_pos", torch.int32), B, Tq, n_h, d, rope_dim, rope_base,
        (d ** -0.5) if scale is None else scale, dt, _ptr(out, "out"),
        _ptr(workspace, "workspace"), ws_bytes, _stream()))


def csa_out_proj_workspace_size(T: int, n_h: int, c: int, groups: int, d_g: int, d: int) -> int:
    return int(_lib.csa_out_proj_workspace_size(T, n_h, c, groups, d_g, d))


def csa_grouped_out_proj(o, W1, W2, y, out, *, workspace=None):
    """Grouped output projection.  o [T, n_h, c] (or [B, Tq, n_h, c]) bf16, W1 [g, d_g, n_h c / g],
    W2 [d, g d_g], y [T, g d_g] and out [T, d] (written), all bf16."""
    if o.dim() == 4:
        o = o.reshape(-1, o.shape[2], o.shape[3])
    T, n_h, c = o.shape
    g, d_g, W = W1.shape
    d = W2.shape[0]
    if g * W != n_h * c or tuple(W2.shape) != (d, g * d_g):
        raise ValueError("W1 must be [g, d_g, n_h c / g] and W2 [d, g d_g]")
    if tuple(y.shape) != (T, g * d_g) or tuple(out.shape) != (T, d):
        raise ValueError("y must be [T, g d_g] and out [T, d]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    bf = torch.bfloat16
    _check(_lib.csa_grouped_out_proj(
        _ptr(o, "o", bf), _ptr(W1, "W1", bf, 3), _ptr(W2, "W2", bf, 2), _ptr(y, "y", bf, 2),
        _ptr(out, "out", bf, 2), T, n_h, c, g, d_g, d, _ptr(workspace, "workspace"), ws_bytes, _stream()))


def cache_ring_slots(m: int, m_hca: int) -> int:
    """Token slots of the tail ring: lcm(m, m')."""
    import math
    return m * m_hca // math.gcd(m, m_hca)


def csa_cache_append(T0, new: dict, tail, E_csa, K_idx, E_hca, W, *, m: int, m_hca: int, K_scale=None,
                     gamma=None, eps: float = 1e-6, rope_dim: int = 0, rope_base: float = 10000.0):
    """Heterogeneous cache append.  T0 [B] int32 (tokens before); new: dict of [B, n_new, width]
    bf16 rows "Ca", "Za", "Cb", "Zb", "ICa", "IZa", "ICb", "IZb", "Ch", "Zh", "Wraw";
    tail [B, lcm(m, m'), 6 c + 4 d_I] bf16; E_csa [B, N_csa, c]; K_idx [B, N_csa, d_I] (bf16,
    float8_e4m3fn with K_scale [B, N_csa], or uint8 MXFP4 [B, N_csa, d_I / 2] with K_scale
    uint8 [B, N_csa, d_I / 32]); E_hca [B, N_hca, c]; W [B, W_cap, c]."""
    names = ("Ca", "Za", "Cb", "Zb", "ICa", "IZa", "ICb", "IZb", "Ch", "Zh", "Wraw")
    B, n_new, c = new["Ca"].shape
    d_I = new["ICa"].shape[2]
    for k in names:
        want = (B, n_new, d_I if k.startswith("I") else c)
        if tuple(new[k].shape) != want or new[k].dtype != torch.bfloat16:
            raise ValueError(f"{k} must be bf16 {want}")
    R = cache_ring_slots(m, m_hca)
    if tuple(tail.shape) != (B, R, 6 * c + 4 * d_I):
        raise ValueError(f"tail must be [B, {R}, {6 * c + 4 * d_I}]")
    N_csa, N_hca, W_cap = E_csa.shape[1], E_hca.shape[1], W.shape[1]
    kd = _dt(K_idx)
    _check(_lib.csa_cache_append(
        B, _ptr(T0, "T0", torch.int32), n_new, c, d_I, m, m_hca, *(_ptr(new[k], k) for k in names),
        _ptr(tail, "tail", torch.bfloat16), _ptr(E_csa, "E_csa", torch.bfloat16), _ptr(K_idx, "K_idx"),
        _ptr(K_scale, "K_scale"), kd, N_csa, _ptr(E_hca, "E_hca", torch.bfloat16), N_hca,
        _ptr(W, "W", torch.bfloat16), W_cap, _ptr(gamma, "gamma", torch.float32), eps, rope_dim, rope_base,
        _stream()))
