"""Exact decoders / round-to-nearest-even encoders for the stored dtypes.

TEST INFRASTRUCTURE (part of the oracle): see ``oracle/__init__.py``.

Written from the format definitions, not from any library routine:

* bfloat16: the upper 16 bits of an IEEE binary32 (1 sign, 8 exponent,
  7 fraction bits, bias 127).
* OCP FP8 E4M3FN: 1 sign, 4 exponent, 3 fraction bits, bias 7;
  e >= 1: (-1)^s 2^(e-7) (1 + f/8); e = 0: (-1)^s 2^-6 (f/8);
  S.1111.111 (0x7F / 0xFF) is NaN; there are no infinities; the largest
  finite magnitude is 448 = S.1111.110.

* OCP Microscaling (MX) formats, v1.0: FP4 E2M1 elements (1 sign, 2 exponent,
  1 mantissa bit, bias 1; e >= 1: (-1)^s 2^(e-1) (1 + m/2); e = 0: (-1)^s m/2;
  no infinities or NaN; largest magnitude 6) and the E8M0 block scale
  (an unsigned exponent: 2^(e - 127); 0xFF is NaN).

The DeepSeek-V4 abstract page (section 3.3) stores KV entries partly in BF16
and partly in FP8, and section 3.6 runs the indexer's QK path in FP4; the
1M-context decode workload stores indexer keys as e4m3 with a per-row scale.
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


# ---------------------------------------------------------------------------
# OCP MX: FP4 E2M1 elements with an E8M0 scale per block of 32
# ---------------------------------------------------------------------------
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest power of two in E2M1 (4 = 2^2)
MX_BLOCK = 32


def e2m1_to_f64(u4) -> np.ndarray:
    """Exact value of FP4 E2M1 codes (0..15), by the closed form."""
    u = np.asarray(u4).astype(np.int64)
    s = (u >> 3) & 1
    e = (u >> 1) & 3
    m = u & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e8m0_to_f64(u8) -> np.ndarray:
    """Exact value of E8M0 scale codes: 2^(code - 127); 255 is NaN."""
    u = np.asarray(u8).astype(np.int64)
    return np.where(u == 255, np.nan, np.ldexp(1.0, u - 127))


def f64_to_e2m1_value(x) -> np.ndarray:
    """RNE rounding to the E2M1 grid with saturation to +-6 (as fp64).  The
    grid has 2 significant bits above 1 and a spacing of 0.5 below it."""
    r = _round_sig(x, 2, 0)
    return np.clip(r, -E2M1_MAX, E2M1_MAX)


def e2m1_code(v) -> np.ndarray:
    """Code of an E2M1-representable value (inverse of ``e2m1_to_f64``; -0.0 -> 8)."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    table = e2m1_to_f64(np.arange(8))           # increasing magnitudes
    idx = np.minimum(np.searchsorted(table, mag), 7)
    if not np.all(table[idx] == mag):
        raise ValueError("not an E2M1 value")
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def mx_quantize_fp4(x) -> tuple[np.ndarray, np.ndarray]:
    """OCP MX conversion of rows to MXFP4, blocks of 32 along the last axis.

    Per block: the shared exponent is floor(log2(max |x|)) - 2 (E2M1's largest
    power of two is 2^2), clamped to E8M0's [-127, 127]; an all-zero block
    takes -127.  Each element is x / 2^shared rounded to E2M1 (RNE, saturated
    to +-6).  The decisions are taken on the given values, which callers
    round to the precision the values are stored or computed in first.
    Returns (element codes uint8 [..., n], scale codes uint8 [..., n / 32]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("the last axis must be a multiple of 32")
    xb = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(xb), axis=-1)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz])).astype(np.int64)
    # log2 may be off by one right at powers of two: correct with exact checks
    e = np.where(nz & (np.ldexp(1.0, e) > amax), e - 1, e)
    e = np.where(nz & (np.ldexp(1.0, e + 1) <= amax), e + 1, e)
    shared = np.where(nz, np.clip(e - E2M1_EMAX, -127, 127), -127)
    y = xb / np.ldexp(1.0, shared)[..., None]
    codes = e2m1_code(f64_to_e2m1_value(y)).reshape(x.shape)
    return codes, (shared + 127).astype(np.uint8)


def mx_fp4_to_f64(codes, scales) -> np.ndarray:
    """Values of MXFP4 rows: element value times its block's scale."""
    v = e2m1_to_f64(codes)
    n = v.shape[-1]
    sc = e8m0_to_f64(scales)
    return (v.reshape(*v.shape[:-1], n // MX_BLOCK, MX_BLOCK) * sc[..., None]).reshape(v.shape)


def unpack_fp4(packed) -> np.ndarray:
    """E2M1 codes from bytes holding two each, the even element in the low nibble."""
    b = np.asarray(packed).astype(np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out
