"""Pins for the oracle's building blocks (CPU only): closed forms,
invariants and library routines that the definitions reduce to."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import decode as od


def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, -3.0, 1e-3, 7.0):
        x = np.full(64, c)
        y = od.rmsnorm(x, np.ones(64), 1e-6)
        assert np.allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(300)
    g = rng.standard_normal(300)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (300,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(od.rmsnorm(x, g, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 16))
    assert np.array_equal(od.rope(x, 0, 1e4), x)
    for pos in (1, 17, 4095, 200000):
        y = od.rope(x, pos, 1e4)
        # each rotated pair (i, i + d/2) keeps its length
        n0 = x[:, :8] ** 2 + x[:, 8:] ** 2
        n1 = y[:, :8] ** 2 + y[:, 8:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 32))
    k = rng.standard_normal((1, 32))
    a = float((od.rope(q, 10, 1e4) @ od.rope(k, 3, 1e4).T)[0, 0])
    b = float((od.rope(q, 107, 1e4) @ od.rope(k, 100, 1e4).T)[0, 0])
    assert abs(a - b) < 1e-10


def test_rope_first_pair_is_plain_rotation():
    # pair 0 turns by exactly pos radians (theta^0 = 1)
    x = np.zeros((1, 8))
    x[0, 0] = 1.0
    y = od.rope(x, 3, 1e4)
    assert np.allclose([y[0, 0], y[0, 4]], [math.cos(3), math.sin(3)], atol=1e-15)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 100)) * 30
    assert np.allclose(od.softmax(z).sum(-1), 1.0, atol=1e-14)


def test_attention_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(4)
    T, Hkv, d = 50, 2, 16
    k = np.repeat(rng.standard_normal((1, Hkv, d)), T, axis=0)
    v = rng.standard_normal((T, Hkv, d))
    q = rng.standard_normal((4, d))
    o = od.attention(q, k, v)
    for h in range(4):
        assert np.allclose(o[h], v[:, h * Hkv // 4].mean(0), atol=1e-13)


def test_attention_dominant_key_and_grouping():
    rng = np.random.default_rng(5)
    T, Hkv, d, Hq = 40, 2, 8, 6
    k = rng.standard_normal((T, Hkv, d)) * 0.01
    v = rng.standard_normal((T, Hkv, d))
    q = np.ones((Hq, d))
    k[17, 0] = 1e3       # dominates for KV head 0 only
    o = od.attention(q, k, v)
    for h in range(Hq):
        g = h * Hkv // Hq   # heads 0..2 -> KV head 0, 3..5 -> KV head 1
        assert g == (0 if h < 3 else 1)
        if g == 0:
            assert np.allclose(o[h], v[17, 0], atol=1e-12)
        else:
            assert not np.allclose(o[h], v[17, 1], atol=1e-3)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(6)
    T, Hkv, d, Hq = 33, 2, 16, 8
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    rep = Hq // Hkv
    kt = torch.from_numpy(np.repeat(k.transpose(1, 0, 2), rep, axis=0))  # [Hq][T][d]
    vt = torch.from_numpy(np.repeat(v.transpose(1, 0, 2), rep, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, :], kt, vt)[:, 0, :]
    assert np.allclose(od.attention(q, k, v), ref.numpy(), atol=1e-13)


def test_attention_split_invariance():
    # log-sum-exp merging of any split of the positions equals the whole
    rng = np.random.default_rng(7)
    T, d = 200, 16
    q = rng.standard_normal(d)
    k = rng.standard_normal((T, d))
    v = rng.standard_normal((T, d))
    s = k @ q / math.sqrt(d)
    whole = od.softmax(s) @ v
    for nsplit in (1, 3, 7, 64, 200):
        parts = np.array_split(np.arange(T), nsplit)
        ms = [s[p].max() for p in parts]
        ls = [np.exp(s[p] - m).sum() for p, m in zip(parts, ms)]
        os_ = [np.exp(s[p] - m) @ v[p] for p, m in zip(parts, ms)]
        M = max(ms)
        L = sum(l * math.exp(m - M) for l, m in zip(ls, ms))
        O = sum(o * math.exp(m - M) for o, m in zip(os_, ms))
        assert np.allclose(O / L, whole, atol=1e-13)


def test_silu_closed_forms():
    assert od.silu(np.array([0.0]))[0] == 0.0
    assert abs(od.silu(np.array([50.0]))[0] - 50.0) < 1e-15
    z = np.linspace(-5, 5, 11)
    assert np.allclose(od.silu(z), z * torch.sigmoid(torch.from_numpy(z)).numpy(), atol=1e-15)


def test_topk_bruteforce_and_ties():
    rng = np.random.default_rng(8)
    for trial in range(50):
        n, k = int(rng.integers(9, 600)), int(rng.integers(1, 9))
        x = np.round(rng.standard_normal(n) * 3, 1)   # many exact ties
        got = list(od.topk_lower_index(x, k))
        # brute force: repeatedly take the first maximum
        rem = list(range(n))
        want = []
        for _ in range(k):
            best = rem[0]
            for i in rem:
                if x[i] > x[best]:
                    best = i
            want.append(best)
            rem.remove(best)
        assert got == want
    assert od.argmax_lower_index(np.array([1.0, 3.0, 3.0, 2.0])) == 1


def test_route_weights_renormalised_and_same_as_logit_topk():
    rng = np.random.default_rng(9)
    r = rng.standard_normal(512) * 2
    sel, w = od.route(r, 8)
    assert abs(w.sum() - 1.0) < 1e-14
    p = od.softmax(r)
    assert list(sel) == list(np.argsort(-p, kind="stable")[:8])
    assert np.all(np.diff(p[sel]) <= 0)
    assert np.allclose(w, p[sel] / p[sel].sum())


def test_quantize_fp8_rows_scale_and_roundtrip():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = od.quantize_fp8_rows(bits)
    wf = oracle.codecs.bf16_to_f64(bits)
    amax = np.abs(wf).max(1)
    assert np.array_equal(scale, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    # the row maximum maps to +-448 exactly or within one rounding of it
    deq = od.dequant_fp8_rows(codes, scale)
    assert np.all(np.abs(deq).max(1) <= 448 * scale * (1 + 1e-6))
    # relative error of E4M3 with round-to-nearest is at most 2^-4 for normals
    big = np.abs(wf) >= scale[:, None] * 2.0 ** -6
    rel = np.abs(deq - wf)[big] / np.abs(wf)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-12
    # torch's converter gives the same codes (all in range by construction)
    y = torch.from_numpy((wf.astype(np.float32) / scale[:, None]).astype(np.float32))
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


def test_quantize_fp8_rows_zero_row():
    bits = np.zeros((2, 32), dtype=np.uint16)
    bits[1, 3] = 0x3F80
    codes, scale = od.quantize_fp8_rows(bits)
    assert scale[0] == 1.0 and np.all(codes[0] == 0)
    assert codes[1, 3] == 0x7E


def test_cache_bulk_prefill_equals_store():
    """OracleCache.prefill_f32 stores what per-position store() stores."""
    from oracle import OracleCache
    rng = np.random.default_rng(9)
    for kv_dtype in ("bf16", "fp8"):
        a = OracleCache(2, 40, 2, 16, kv_dtype)
        b = OracleCache(2, 40, 2, 16, kv_dtype)
        if kv_dtype == "fp8":
            a.scales = b.scales = np.array([[[2.0**-3, 0.5], [1.0, 0.75]]] * 2, dtype=np.float32)
        k = rng.standard_normal((40, 2, 16)).astype(np.float32) * 7
        v = rng.standard_normal((40, 2, 16)).astype(np.float32) * 7
        for li in range(2):
            a.prefill_f32(li, 0, k, v)
            for p in range(40):
                b.store(li, p, k[p], v[p])
            assert np.array_equal(a.k[li], b.k[li]) and np.array_equal(a.v[li], b.v[li])
            ka, va = a.read(li, 40)
            kb, vb = b.read(li, 40)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
