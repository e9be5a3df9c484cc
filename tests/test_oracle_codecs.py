"""Pins for the oracle's number formats (CPU only).

Each decoder is checked exhaustively against the format specification's
printed values (tests/golden) and against torch's own converters; each
encoder against a brute-force nearest search over the decoded code table.
"""
import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------- BF16

def test_bf16_decode_matches_struct():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = codecs.bf16_to_f64(bits)
    for b in range(0, 1 << 16, 97):
        ref = struct.unpack("<f", struct.pack("<I", b << 16))[0]
        if math.isnan(ref):
            assert math.isnan(got[b])
        else:
            assert got[b] == ref


def test_bf16_rne_matches_torch_and_bruteforce():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-35).astype(np.float32),
    ])
    # exact ties: low 16 bits 0x8000, both parities
    u = (rng.integers(0, 1 << 15, 4000).astype(np.uint32) << 16) | 0x8000
    u[:2000] |= 0x3F800000
    ties = u.view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    got = codecs.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # brute force on a sample: the nearer of the two bracketing BF16 values
    for xi, gi in zip(x[:3000], got[:3000]):
        lo = np.uint16(np.float32(xi).view(np.uint32) >> 16)
        cands = [lo, np.uint16(lo + 1)]
        vals = [codecs.bf16_to_f64(c) for c in cands]
        dist = [abs(float(v) - float(xi)) for v in vals]
        if dist[0] < dist[1]:
            want = cands[0]
        elif dist[1] < dist[0]:
            want = cands[1]
        else:
            want = cands[0] if int(cands[0]) % 2 == 0 else cands[1]
        assert gi == want


def test_bf16_nan_stays_nan():
    out = codecs.f32_to_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(codecs.bf16_to_f64(out)))


# --------------------------------------------------------------------------- FP8

def test_fp8_landmarks_from_spec():
    for code, val in _read_golden("fp8_e4m3fn_landmarks.txt"):
        got = codecs.fp8e4m3_to_f64(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = codecs.fp8e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.all(both_nan | (got == ref))
    assert np.sum(np.isnan(got)) == 2
    # 254 finite codes, 253 distinct values (+0 and -0 compare equal)
    assert np.unique(got[~np.isnan(got)]).size == 253
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0)  # monotone over 0x00..0x7E


def test_fp8_encode_bruteforce_nearest_even():
    table = codecs.fp8e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    rng = np.random.default_rng(5)
    mags = np.concatenate([
        np.abs(rng.standard_normal(4000)) * 64,
        rng.uniform(0, 2 ** -6, 2000),
        rng.uniform(400, 520, 500),
        (table[:-1] + table[1:]) / 2,      # every midpoint (ties)
        table,
    ]).astype(np.float32)
    x = np.concatenate([mags, -mags])
    got = codecs.f32_to_fp8e4m3(x)
    for xi, gi in zip(x, got):
        a = abs(float(xi))
        if a >= 448:
            want = 0x7E
        else:
            dist = np.abs(table - a)
            best = np.flatnonzero(dist == dist.min())
            want = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        if math.copysign(1.0, float(xi)) < 0:
            want |= 0x80
        assert gi == want, (xi, gi, want)


def test_fp8_encode_matches_torch_in_range():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(50000) * 50).astype(np.float32)
    x = x[np.abs(x) < 448]
    got = codecs.f32_to_fp8e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_fp8_encode_saturates_and_nan():
    got = codecs.f32_to_fp8e4m3(np.array([1e6, -1e6, 449.0, 464.0, np.inf, np.nan], dtype=np.float32))
    assert list(got[:5]) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E]
    assert got[5] & 0x7F == 0x7F


# --------------------------------------------------------------------------- MXFP4

def test_e2m1_table_from_spec():
    rows = _read_golden("e2m1_values.txt")
    assert len(rows) == 8
    for code, val in rows:
        c = int(code)
        assert codecs.e2m1_to_f64(np.array([c]))[0] == float(val)
        neg = codecs.e2m1_to_f64(np.array([c | 8]))[0]
        assert neg == -float(val) and math.copysign(1, neg) == -1


def test_e8m0_all_bytes():
    e = np.arange(256)
    v = codecs.e8m0_to_f64(e)
    assert math.isnan(v[255])
    for i in range(255):
        assert v[i] == math.ldexp(1.0, i - 127)


def test_mxfp4_all_products_and_layout():
    # all 16 codes x all 255 finite scales, plus the nibble order of a row
    codes = np.zeros((255, 16), dtype=np.uint8)     # 32 elements per row
    for j in range(16):
        codes[:, j] = (j & 0xF) | (((15 - j) & 0xF) << 4)
    scales = np.arange(255, dtype=np.uint8)[:, None]
    out = codecs.mxfp4_to_f64(codes, scales)
    tbl = {int(c): float(v) for c, v in _read_golden("e2m1_values.txt")}

    def val(c):
        return (-1.0 if c & 8 else 1.0) * tbl[c & 7]

    for e in (0, 1, 2, 100, 120, 121, 122, 127, 200, 254):
        for j in range(16):
            assert out[e, 2 * j] == val(j) * math.ldexp(1.0, e - 127)
            assert out[e, 2 * j + 1] == val(15 - j) * math.ldexp(1.0, e - 127)


def test_fp8_bulk_codec_equals_direct():
    """The table forms used for large caches compute the same functions:
    every (top 13 bits, sticky) class of binary32 with several low-bit
    patterns, plus random values; decoding of all 256 codes with scales."""
    rng = np.random.default_rng(5)
    top = np.arange(1 << 13, dtype=np.uint32) << np.uint32(19)
    lows = np.array([0, 1, 0x40000, 0x7FFFF, 0x12345, 0x00100], dtype=np.uint32)
    bits = (top[:, None] | lows[None, :]).reshape(-1)
    rnd = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([bits, rnd]).view(np.float32)
    with np.errstate(invalid="ignore"):
        direct = codecs.f32_to_fp8e4m3(x)
    assert np.array_equal(codecs.f32_to_fp8e4m3_bulk(x), direct)
    big = (rng.standard_normal(5_000_000).astype(np.float32) * 64)   # takes the threaded path
    assert np.array_equal(codecs.f32_to_fp8e4m3_bulk(big), codecs.f32_to_fp8e4m3(big))
    c = rng.integers(0, 256, (300, 4, 16), dtype=np.uint8)
    sc = np.array([[2.0**-6], [0.75], [3.0], [1.0]])
    assert np.array_equal(codecs.fp8e4m3_to_f64_bulk(c, sc), codecs.fp8e4m3_to_f64(c) * sc[None],
                          equal_nan=True)
    assert np.array_equal(codecs.fp8e4m3_to_f64_bulk(c), codecs.fp8e4m3_to_f64(c), equal_nan=True)


def test_mxfp4_bulk_equals_direct():
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 256, (40, 64), dtype=np.uint8)
    scales = rng.integers(0, 256, (40, 4), dtype=np.uint8)
    scales[0, :] = [0, 1, 254, 255]
    a = codecs.mxfp4_to_f64(codes, scales)
    b = codecs.mxfp4_to_f64_bulk(codes, scales)
    assert np.array_equal(a, b, equal_nan=True)
