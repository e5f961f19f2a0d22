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
    "CsaError", "LIB_PATH", "abi_version", "csa_compress", "csa_compress_batch", "csa_index_score",
    "csa_topk",
    "csa_topk_workspace_size", "csa_sparse_mqa", "hca_dense_mqa", "csa_mqa_workspace_size",
    "CSA_F32", "CSA_BF16", "CSA_FP8_E4M3",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
CSA_F32, CSA_BF16, CSA_FP8_E4M3 = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m long_context_attention_02_amd.build` "
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
_lib.csa_compress.argtypes = [_P, _P, _P, _P, _I, _I, _L, _L, _L, _L, _I, _I, _I, _L, _L, _P, _F, _I,
                              _F, _L, _L, _P, _I, _P, _L, _L, _P]


class _CompressJob(ctypes.Structure):
    """csa_compress_job of include/csa.h (C layout, natural alignment)."""
    _fields_ = [("C_a", _P), ("Z_a", _P), ("C_b", _P), ("Z_b", _P), ("in_dtype", _I), ("B", _I),
                ("R", _L), ("in_batch_stride", _L), ("tok_base", _L), ("T", _L),
                ("c", _I), ("m", _I), ("overlap", _I), ("s_begin", _L), ("s_end", _L),
                ("gamma", _P), ("eps", _F), ("rope_dim", _I), ("rope_base", _F),
                ("pos_stride", _L), ("pos_offset", _L), ("E", _P), ("out_dtype", _I),
                ("E_scale", _P), ("out_batch_stride", _L), ("out_ring", _L)]


_lib.csa_compress_batch.restype = _I
_lib.csa_compress_batch.argtypes = [ctypes.POINTER(_CompressJob), _I, _P]
_lib.csa_index_score.restype = _I
_lib.csa_index_score.argtypes = [_P, _I, _P, _P, _I, _P, _P, _I, _I, _I, _I, _L, _I, _P, _P]
_lib.csa_topk_workspace_size.restype = _S
_lib.csa_topk_workspace_size.argtypes = [_I, _I, _L, _I]
_lib.csa_topk.restype = _I
_lib.csa_topk.argtypes = [_P, _P, _I, _I, _L, _I, _I, _P, _P, _P, _S, _P]
_lib.csa_mqa_workspace_size.restype = _S
_lib.csa_mqa_workspace_size.argtypes = [_I, _I, _I, _I, _L]
_lib.csa_sparse_mqa.restype = _I
_lib.csa_sparse_mqa.argtypes = [_P, _P, _F, _P, _L, _P, _I, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I,
                                _F, _F, _I, _P, _P, _S, _P]
_lib.hca_dense_mqa.restype = _I
_lib.hca_dense_mqa.argtypes = [_P, _P, _F, _P, _L, _I, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _F,
                               _F, _I, _P, _P, _S, _P]


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


_DT = {torch.float32: CSA_F32, torch.bfloat16: CSA_BF16, torch.float8_e4m3fn: CSA_FP8_E4M3}


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
                   E_scale=None, out_ring: int = 0):
    """The C arguments of one compression (without the stream), in csa_compress order."""
    B, R, c = C_a.shape
    for name, t in (("Z_a", Z_a), ("C_b", C_b), ("Z_b", Z_b)):
        if t is not None and (t.shape != C_a.shape or t.dtype != C_a.dtype):
            raise ValueError(f"{name} must match C_a in shape and dtype")
    if E.dim() != 3 or E.shape[0] != B or E.shape[2] != c:
        raise ValueError("E must be [B, rows, c]")
    if E.shape[1] < (out_ring if out_ring > 0 else s_end):
        raise ValueError("E has fewer rows than the entries written")
    if E_scale is not None and tuple(E_scale.shape) != (B, E.shape[1]):
        raise ValueError("E_scale must be [B, rows]")
    return (_ptr(C_a, "C_a", dims=3), _ptr(Z_a, "Z_a"), _ptr(C_b, "C_b"), _ptr(Z_b, "Z_b"), _dt(C_a),
            B, R, R * c, tok_base, T, c, m, overlap, s_begin, s_end,
            _ptr(gamma, "gamma", torch.float32), eps, rope_dim, rope_base,
            m if pos_stride is None else pos_stride, pos_offset,
            _ptr(E, "E"), _dt(E), _ptr(E_scale, "E_scale", torch.float32), E.shape[1] * c, out_ring)


def csa_compress(C_a, Z_a, C_b, Z_b, E, **kw):
    """a1.  C_a/Z_a/C_b/Z_b: [B, R, c] (Z may be None; C_b None when overlap=0),
    E: [B, rows, c] float32 / bfloat16 / float8_e4m3fn, E_scale: [B, rows] fp32
    for fp8 output.  Row r of the candidates is token tok_base + r.  Keywords:
    T, m, overlap, s_begin, s_end (required); tok_base, gamma, eps, rope_dim,
    rope_base, pos_stride (default m), pos_offset, E_scale, out_ring."""
    _check(_lib.csa_compress(*_compress_args(C_a, Z_a, C_b, Z_b, E, **kw), _stream()))


def csa_compress_batch(jobs):
    """a1, several compressions in one launch.  ``jobs`` is a list of
    (C_a, Z_a, C_b, Z_b, E, kwargs) with the arguments of csa_compress; the
    outputs equal those of the separate calls."""
    arr = (_CompressJob * max(len(jobs), 1))()
    for q, (C_a, Z_a, C_b, Z_b, E, kw) in enumerate(jobs):
        arr[q] = _CompressJob(*_compress_args(C_a, Z_a, C_b, Z_b, E, **kw))
    _check(_lib.csa_compress_batch(arr, len(jobs), _stream()))


def csa_index_score(q_I, w_I, K_I, q_pos, I_out, *, m: int, K_scale=None):
    """a2.  q_I [B, Tq, H, dI], w_I [B, Tq, H] fp32, K_I [B, N, dI],
    q_pos [B, Tq] int32, I_out [B, Tq, N] fp32, K_scale [B, N] for fp8 keys."""
    B, Tq, H, dI = q_I.shape
    N = K_I.shape[1]
    if tuple(w_I.shape) != (B, Tq, H) or K_I.shape[0] != B or K_I.shape[2] != dI:
        raise ValueError("shape mismatch among q_I, w_I, K_I")
    if K_scale is not None and tuple(K_scale.shape) != (B, N):
        raise ValueError("K_scale must be [B, N]")
    if tuple(I_out.shape) != (B, Tq, N) or tuple(q_pos.shape) != (B, Tq):
        raise ValueError("I_out must be [B, Tq, N] and q_pos [B, Tq]")
    _check(_lib.csa_index_score(
        _ptr(q_I, "q_I", dims=4), _dt(q_I), _ptr(w_I, "w_I", torch.float32), _ptr(K_I, "K_I", dims=3),
        _dt(K_I), _ptr(K_scale, "K_scale", torch.float32), _ptr(q_pos, "q_pos", torch.int32),
        B, Tq, H, dI, N, m, _ptr(I_out, "I_out", torch.float32), _stream()))


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


def _mqa_common(q, E, W, q_pos, out, sink, gamma_q):
    B, Tq, n_h, d = q.shape
    if E.dim() != 3 or E.shape[0] != B or E.shape[2] != d or E.dtype != q.dtype:
        raise ValueError("E must be [B, N, d] with q's dtype")
    if W is not None and (W.dim() != 3 or W.shape[0] != B or W.shape[2] != d or W.dtype != q.dtype):
        raise ValueError("W must be [B, W_cap, d] with q's dtype")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if tuple(q_pos.shape) != (B, Tq):
        raise ValueError("q_pos must be [B, Tq]")
    if sink is not None and tuple(sink.shape) != (n_h,):
        raise ValueError("sink must be [n_h]")
    if gamma_q is not None and tuple(gamma_q.shape) != (d,):
        raise ValueError("gamma_q must be [d]")
    return B, Tq, n_h, d


def csa_sparse_mqa(q, E, idx, W, q_pos, out, *, n_win: int, sink=None, gamma_q=None, eps: float = 1e-6,
                   rope_dim: int = 0, rope_base: float = 10000.0, scale: float | None = None,
                   workspace=None):
    """a4.  q [B, Tq, n_h, d], E [B, N, d], idx [B, Tq, k] int32, W [B, W_cap, d]
    or None, q_pos [B, Tq] int32, out like q; sink [n_h], gamma_q [d] fp32."""
    B, Tq, n_h, d = _mqa_common(q, E, W, q_pos, out, sink, gamma_q)
    k = idx.shape[2]
    if tuple(idx.shape[:2]) != (B, Tq):
        raise ValueError("idx must be [B, Tq, k]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.csa_sparse_mqa(
        _ptr(q, "q", dims=4), _ptr(gamma_q, "gamma_q", torch.float32), eps, _ptr(E, "E"), E.shape[1],
        _ptr(idx, "idx", torch.int32, 3), k, _ptr(W, "W"), 0 if W is None else W.shape[1], n_win,
        _ptr(sink, "sink", torch.float32), _ptr(q_pos, "q_pos", torch.int32), B, Tq, n_h, d,
        rope_dim, rope_base, (d ** -0.5) if scale is None else scale, _dt(q), _ptr(out, "out"),
        _ptr(workspace, "workspace"), ws_bytes, _stream()))


def hca_dense_mqa(q, E, W, q_pos, out, *, m: int, n_win: int, sink=None, gamma_q=None, eps: float = 1e-6,
                  rope_dim: int = 0, rope_base: float = 10000.0, scale: float | None = None,
                  workspace=None):
    """a5.  As csa_sparse_mqa over every visible entry s < floor((i+1)/m)."""
    B, Tq, n_h, d = _mqa_common(q, E, W, q_pos, out, sink, gamma_q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.hca_dense_mqa(
        _ptr(q, "q", dims=4), _ptr(gamma_q, "gamma_q", torch.float32), eps, _ptr(E, "E"), E.shape[1], m,
        _ptr(W, "W"), 0 if W is None else W.shape[1], n_win, _ptr(sink, "sink", torch.float32),
        _ptr(q_pos, "q_pos", torch.int32), B, Tq, n_h, d, rope_dim, rope_base,
        (d ** -0.5) if scale is None else scale, _dt(q), _ptr(out, "out"),
        _ptr(workspace, "workspace"), ws_bytes, _stream()))
