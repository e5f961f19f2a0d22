"""Test helpers: exact decoding of device tensors for the oracle and error metrics."""
from __future__ import annotations

import numpy as np
import torch

from oracle import codecs as oc


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a tensor's stored bytes (decoded by the oracle's codecs)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype == torch.bfloat16:
        return oc.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float8_e4m3fn:
        return oc.e4m3_to_f64(t.view(torch.uint8).numpy())
    if t.dtype in (torch.int32, torch.int64):
        return t.numpy().astype(np.int64)
    raise TypeError(t.dtype)


def row_rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis) of ||x - ref||_inf / ||ref||_inf."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, np.shape(x)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.max(np.abs(x - ref), axis=1)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(num / den)) if len(num) else 0.0


def e4m3_ulp(y: np.ndarray) -> np.ndarray:
    """Spacing of e4m3fn values around |y| (2^-9 in the subnormal range)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    return np.ldexp(1.0, (e - 3).astype(np.int64))


TOL_BF16 = 2e-2   # relative tolerance for bf16 outputs
TOL_F32 = 1e-5    # relative tolerance for fp32 outputs
