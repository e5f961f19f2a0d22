"""Exact decoders / round-to-nearest-even encoders for the stored dtypes.

TEST INFRASTRUCTURE (part of the oracle): see ``oracle/__init__.py``.

Written from the format definitions, not from any library routine:

* bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent,
  7 fraction bits, bias 127).
* OCP FP8 E4M3FN: 1 sign, 4 exponent, 3 fraction bits, bias 7;
  e >= 1: (-1)^s 2^(e-7) (1 + f/8); e = 0: (-1)^s 2^-6 (f/8);
  S.1111.111 (0x7F / 0xFF) is NaN; there are no infinities; the largest
  finite magnitude is 448 = S.1111.110.

The DeepSeek-V4 abstract page (section 3.3) stores KV entries partly in BF16
and partly in FP8; the 1M-context decode workload stores indexer keys as e4m3
with a per-row scale.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(u16) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16 array)."""
    u = np.asarray(u16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def e4m3_to_f64(u8) -> np.ndarray:
    """Exact value of OCP e4m3fn codes (uint8 array), by the closed form."""
    u = np.asarray(u8).astype(np.int64)
    s = (u >> 7) & 1
    e = (u >> 3) & 0xF
    f = u & 0x7
    mag = np.where(e == 0, np.ldexp(f / 8.0, -6), np.ldexp(1.0 + f / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((u & 0x7F) == 0x7F, np.nan, val)


def _round_sig(x, sig_bits: int, emin: int) -> np.ndarray:
    """Round fp64 values to `sig_bits` significant bits (RNE), with gradual
    underflow below 2**emin (the smallest normal).  No overflow handling."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # log2 can be off by one right at powers of two: correct with exact checks
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, emin)
    ulp_exp = (e - (sig_bits - 1)).astype(np.int64)
    q = np.rint(np.ldexp(x, -ulp_exp))          # np.rint: round half to even
    return np.ldexp(q, ulp_exp)


def f64_to_bf16_value(x) -> np.ndarray:
    """RNE rounding of fp64 values to the nearest bfloat16 value (as fp64)."""
    r = _round_sig(x, 8, -126)
    big = np.abs(r) > 3.3895313892515355e38     # beyond the largest finite bf16
    return np.where(big, np.copysign(np.inf, r), r)


def f64_to_e4m3_value(x) -> np.ndarray:
    """RNE rounding to e4m3fn with saturation to +-448 (as fp64)."""
    r = _round_sig(x, 4, -6)
    return np.clip(r, -448.0, 448.0)


def e4m3_code(v) -> np.ndarray:
    """Code of an e4m3fn-representable value (inverse of ``e4m3_to_f64``)."""
    v = np.asarray(v, dtype=np.float64)
    table = e4m3_to_f64(np.arange(256))
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v = v.reshape(-1)
    flat_o = out.reshape(-1)
    for n, val in enumerate(flat_v):
        hits = np.nonzero(table == val)[0]
        if len(hits) == 0:
            raise ValueError(f"{val} is not an e4m3fn value")
        if val == 0.0:
            hits = [0x80 if np.signbit(val) else 0x00]
        flat_o[n] = hits[0]
    return out
