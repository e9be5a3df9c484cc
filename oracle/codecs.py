"""Number formats of the decode path, from their definitions (float64 math).

TEST INFRASTRUCTURE: see the package docstring.

* BF16: the upper 16 bits of an IEEE-754 binary32.
* FP8 E4M3FN (OCP 8-bit floating point specification): 1 sign, 4 exponent
  bits with bias 7, 3 mantissa bits; subnormals m * 2^-9; largest finite
  value 448; codes 0x7F / 0xFF are NaN; no infinities.  The pages only say
  "FP8" / "fp8_e4m3" (163.com Ling-3.0-flash article, online FP8 LM head
  section; wmrh.cn Kimi-K3 report, test-environment table); E4M3FN is the
  reading taken.
* MXFP4 (OCP Microscaling formats specification): E2M1 elements (1 sign,
  2 exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6)
  sharing one E8M0 scale (2^(e-127), e = 255 is NaN) per block of 32.
  Element 2i sits in the low nibble of byte i.
"""
from __future__ import annotations

import os

import numpy as np

# --------------------------------------------------------------------------
# BF16
# --------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16(x) -> np.ndarray:
    """Round binary32 values to BF16 bit patterns, nearest, ties to even.

    The two candidates are the BF16 numbers on either side of x; the nearer
    one wins, and on a tie the one with an even last mantissa bit.  NaN maps
    to a quiet NaN with the same sign.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lo = (u >> np.uint64(16)).astype(np.uint64)          # truncated candidate
    rem = u & np.uint64(0xFFFF)                           # dropped bits
    half = np.uint64(0x8000)
    up = (rem > half) | ((rem == half) & ((lo & np.uint64(1)) == np.uint64(1)))
    out = (lo + up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        sign = (u >> np.uint64(31)).astype(np.uint16) << np.uint16(15)
        out = np.where(nan, sign | np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


def round_to_bf16(x) -> np.ndarray:
    """A float64 value as the decode path stores it in a BF16 cache: first
    to binary32 (the precision the GPU holds it in), then to BF16."""
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))


# --------------------------------------------------------------------------
# FP8 E4M3FN
# --------------------------------------------------------------------------

FP8_MAX = 448.0


def fp8e4m3_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = s * np.where(e == 0, sub, nor)
    return np.where((e == 15) & (m == 7), np.nan, v)


def _round_half_even(y: np.ndarray) -> np.ndarray:
    return np.round(y)  # numpy rounds halves to even


def f32_to_fp8e4m3(x) -> np.ndarray:
    """binary32 -> E4M3FN code, nearest with ties to even, saturating at 448.

    Magnitudes below 2^-6 are multiples of 2^-9 after rounding (subnormal
    grid, mantissa 8 becomes the smallest normal); above, the exponent is
    floor(log2|x|) and the mantissa is rounded to 3 bits, carrying into the
    exponent when it rounds up to 2.  Anything beyond 448 (including values
    that would round past it, and infinities) is clamped to 448.
    NaN -> 0x7F with sign.
    """
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(f)
    a = np.abs(f)
    nan = np.isnan(f)
    a = np.where(nan, 0.0, a)
    a = np.where(np.isinf(a), 2.0 * FP8_MAX, a)      # saturates below
    code = np.zeros(a.shape, dtype=np.int64)

    small = a < 2.0 ** -6
    q = _round_half_even(a * 2.0 ** 9).astype(np.int64)      # 0..8
    code = np.where(small, q, code)

    big = ~small
    mant, ex = np.frexp(np.where(big, a, 1.0))                 # a = mant * 2^ex, mant in [0.5,1)
    e = ex.astype(np.int64) - 1                                # a = (2*mant) * 2^e
    frac = 2.0 * mant - 1.0                                    # in [0, 1)
    m = _round_half_even(frac * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    sat = (e > 8) | ((e == 8) & (m > 6))
    e = np.where(sat, 8, e)
    m = np.where(sat, 6, m)
    code = np.where(big, ((e + 7) << 3) | m, code)

    code = np.where(nan, 0x7F, code)
    code = code | np.where(sign, 0x80, 0)
    return code.astype(np.uint8)


# Bulk forms of the two FP8 functions above, for caches of hundreds of
# millions of values.  They compute exactly the same function:
#   * decoding looks the code up in the 256 values fp8e4m3_to_f64 gives;
#   * encoding looks up the code that f32_to_fp8e4m3 gives for a binary32
#     with the same top 13 bits (sign, exponent, 3 mantissa bits, the next
#     bit) and the same "any lower bit set" flag.  Those 14 bits decide the
#     result: E4M3FN keeps at most 3 mantissa bits, so rounding to nearest
#     even needs the kept bits, the next one and whether anything below is
#     non-zero; at smaller exponents the rounding point only moves up into
#     the top 13 bits; NaN and infinity differ in the mantissa, which the
#     14 bits also tell apart.


def _fp8_tables():
    global _FP8_ENC, _FP8_DEC
    if _FP8_ENC is None:
        top = np.arange(1 << 13, dtype=np.uint32) << 19
        enc = np.empty((1 << 13, 2), dtype=np.uint8)
        enc[:, 0] = f32_to_fp8e4m3(top.view(np.float32))
        enc[:, 1] = f32_to_fp8e4m3((top | np.uint32(1)).view(np.float32))
        _FP8_ENC = enc.reshape(-1)
        _FP8_DEC = fp8e4m3_to_f64(np.arange(256, dtype=np.uint8))
    return _FP8_ENC, _FP8_DEC


_FP8_ENC = None
_FP8_DEC = None


def _chunked(fn, x: np.ndarray, out_dtype, chunk: int = 1 << 22) -> np.ndarray:
    flat = np.ascontiguousarray(x).reshape(-1)
    out = np.empty(flat.shape, dtype=out_dtype)
    if flat.size <= chunk:
        out[:] = fn(flat)
        return out.reshape(np.shape(x))
    from concurrent.futures import ThreadPoolExecutor
    starts = range(0, flat.size, chunk)

    def run(i):
        out[i:i + chunk] = fn(flat[i:i + chunk])

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(run, starts))
    return out.reshape(np.shape(x))


def f32_to_fp8e4m3_bulk(x) -> np.ndarray:
    """f32_to_fp8e4m3 by table, for large arrays."""
    enc, _ = _fp8_tables()

    def one(a):
        b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
        return enc[((b >> np.uint32(19)) << np.uint32(1)) | ((b & np.uint32(0x7FFFF)) != 0)]

    return _chunked(one, np.asarray(x, dtype=np.float32), np.uint8)


def fp8e4m3_to_f64_bulk(codes, scale=None) -> np.ndarray:
    """fp8e4m3_to_f64 by table, for large arrays; optionally times `scale`
    (broadcast against the codes' trailing axes)."""
    _, dec = _fp8_tables()
    c = np.asarray(codes, dtype=np.uint8)
    if scale is None:
        return _chunked(lambda a: dec[a], c, np.float64)
    sc = np.broadcast_to(np.asarray(scale, dtype=np.float64), c.shape[-2:])

    def one_row_block(a):
        return (dec[a].reshape(-1, *c.shape[-2:]) * sc).reshape(-1)

    per = int(np.prod(c.shape[-2:]))
    return _chunked(one_row_block, c, np.float64, chunk=max(per, (1 << 22) // per * per))


# --------------------------------------------------------------------------
# MXFP4: E2M1 elements with an E8M0 scale per 32
# --------------------------------------------------------------------------


def e2m1_to_f64(nibbles) -> np.ndarray:
    c = np.asarray(nibbles, dtype=np.int64) & 0xF
    s = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    v = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return s * v


def e8m0_to_f64(bytes_) -> np.ndarray:
    e = np.asarray(bytes_, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


def mxfp4_to_f64(codes, scales) -> np.ndarray:
    """Dequantise a [rows][cols/2] code array with [rows][cols/32] scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    el = np.empty((rows, cols), dtype=np.float64)
    el[:, 0::2] = e2m1_to_f64(codes & 0xF)
    el[:, 1::2] = e2m1_to_f64(codes >> 4)
    sc = e8m0_to_f64(scales).reshape(rows, cols // 32)
    return (el.reshape(rows, cols // 32, 32) * sc[:, :, None]).reshape(rows, cols)


# Bulk form of mxfp4_to_f64 for whole expert matrices: the same products,
# looked up in the 16 x 256 table of E2M1 value times E8M0 scale that the
# two functions above give.
_MX_TAB = None


def mxfp4_to_f64_bulk(codes, scales) -> np.ndarray:
    global _MX_TAB
    if _MX_TAB is None:
        _MX_TAB = (e2m1_to_f64(np.arange(16))[None, :] * e8m0_to_f64(np.arange(256))[:, None]).reshape(-1)
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    cols = 2 * half
    sc = np.asarray(scales, dtype=np.uint8).reshape(rows, cols // 32).astype(np.int32) << 4
    nib = np.empty((rows, cols), dtype=np.int32)
    nib[:, 0::2] = codes & 0xF
    nib[:, 1::2] = codes >> 4
    idx = (nib.reshape(rows, cols // 32, 32) + sc[:, :, None]).reshape(rows, cols)
    return _MX_TAB[idx]
