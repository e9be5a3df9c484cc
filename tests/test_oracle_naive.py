"""A second, naive forward (pure-Python loops over floats) on tiny shapes,
checked against the oracle's vectorised step.

The naive model is written independently of ``oracle``: scalar loops, the
``math`` module, torch's own BF16/FP8 converters for cache rounding, and the
spec's E2M1 table for MXFP4.  A dropped term, a wrong sign or index, a
transposed operand or a mis-grouped head in either implementation makes
them disagree.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import OracleCache, OracleModel, quantize_fp8_rows
from synth import gen
from synth.configs import DecodeConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e2m1_table():
    t = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                t[int(c)] = float(v)
                t[int(c) | 8] = -float(v)
    return t


E2M1 = _e2m1_table()


def bf(bits):
    return torch.tensor(int(bits) & 0xFFFF, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).item()


def mat(bits2d):
    return [[bf(b) for b in row] for row in bits2d]


def mxfp4_mat(codes, scales):
    rows = []
    for r in range(codes.shape[0]):
        row = []
        for j in range(codes.shape[1] * 2):
            byte = int(codes[r, j // 2])
            nib = byte & 0xF if j % 2 == 0 else byte >> 4
            row.append(E2M1[nib] * math.ldexp(1.0, int(scales[r, j // 32]) - 127))
        rows.append(row)
    return rows


def matvec(W, x):
    out = []
    for row in W:
        s = 0.0
        for w, xi in zip(row, x):
            s += w * xi
        out.append(s)
    return out


def rms(x, eps, g):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def rot(vec, pos, theta):
    d = len(vec)
    h = d // 2
    out = list(vec)
    for i in range(h):
        a = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i] * s + vec[i + h] * c
    return out


def cache_round(x, kv_dtype, scale):
    t = torch.tensor(x, dtype=torch.float64).to(torch.float32)
    if kv_dtype == "bf16":
        return t.to(torch.bfloat16).to(torch.float64).tolist()
    y = (t / torch.tensor(scale, dtype=torch.float32)).to(torch.float8_e4m3fn)
    return (y.to(torch.float64) * float(scale)).tolist()


class Naive:
    def __init__(self, cfg, T, experts=None, lm=None):
        self.cfg = cfg
        self.L = cfg.n_layers
        self.W = {k: (mat(v) if v.ndim == 2 else [bf(b) for b in v]) for k, v in T.items()}
        if lm is not None:
            codes, sc = lm
            self.W["lm_head"] = [[torch.tensor(int(c), dtype=torch.uint8).view(torch.float8_e4m3fn).item() * float(sc[r])
                                  for c in codes[r]] for r in range(codes.shape[0])]
        self.experts = experts
        self.K = [[None] * cfg.max_pos for _ in range(self.L)]
        self.V = [[None] * cfg.max_pos for _ in range(self.L)]
        self.scales = None

    def ffn(self, li, xn):
        cfg = self.cfg

        def one(G, U, D):
            g = matvec(G, xn)
            u = matvec(U, xn)
            h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
            return matvec(D, h)

        if not cfg.is_moe:
            return one(self.W[f"l{li}.w_gate"], self.W[f"l{li}.w_up"], self.W[f"l{li}.w_down"])
        r = matvec(self.W[f"l{li}.w_router"], xn)
        m = max(r)
        e = [math.exp(v - m) for v in r]
        z = sum(e)
        p = [v / z for v in e]
        chosen = []
        for _ in range(cfg.top_k):
            best = None
            for i in range(len(p)):
                if i in chosen:
                    continue
                if best is None or p[i] > p[best]:
                    best = i
            chosen.append(best)
        tot = sum(p[i] for i in chosen)
        y = [0.0] * len(xn)
        mf = cfg.moe_ffn
        for i in chosen + [cfg.n_experts + s for s in range(cfg.n_shared)]:
            gu = mxfp4_mat(*self.experts(li, i, "gate_up"))
            dn = mxfp4_mat(*self.experts(li, i, "down"))
            o = one(gu[:mf], gu[mf:], dn)
            wgt = p[i] / tot if i < cfg.n_experts else 1.0
            y = [a + wgt * b for a, b in zip(y, o)]
        return y

    def step(self, token, pos):
        cfg = self.cfg
        d, Hq, Hkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
        x = list(self.W["embed"][token])
        for li in range(self.L):
            xn = rms(x, cfg.rms_eps, self.W[f"l{li}.attn_norm"])
            q = matvec(self.W[f"l{li}.wq"], xn)
            k = matvec(self.W[f"l{li}.wk"], xn)
            v = matvec(self.W[f"l{li}.wv"], xn)
            qh = [rot(q[h * d:(h + 1) * d], pos, cfg.rope_theta) for h in range(Hq)]
            kh = [rot(k[g * d:(g + 1) * d], pos, cfg.rope_theta) for g in range(Hkv)]
            vh = [v[g * d:(g + 1) * d] for g in range(Hkv)]
            sk = self.scales[li, :, 0] if self.scales is not None else [1.0] * Hkv
            sv = self.scales[li, :, 1] if self.scales is not None else [1.0] * Hkv
            self.K[li][pos] = [cache_round(kh[g], cfg.kv_dtype, sk[g]) for g in range(Hkv)]
            self.V[li][pos] = [cache_round(vh[g], cfg.kv_dtype, sv[g]) for g in range(Hkv)]
            att = []
            win = cfg.layer_window[li] if cfg.layer_window else 0
            first = pos - win + 1 if win > 0 and pos - win + 1 > 0 else 0   # the last `win` positions
            for h in range(Hq):
                g = h * Hkv // Hq
                sc = []
                for t in range(first, pos + 1):
                    kt = self.K[li][t][g]
                    sc.append(sum(a * b for a, b in zip(qh[h], kt)) / math.sqrt(d))
                m = max(sc)
                w = [math.exp(s - m) for s in sc]
                z = sum(w)
                o = [0.0] * d
                for i, t in enumerate(range(first, pos + 1)):
                    vt = self.V[li][t][g]
                    for j in range(d):
                        o[j] += w[i] / z * vt[j]
                att.extend(o)
            y = matvec(self.W[f"l{li}.wo"], att)
            x = [a + b for a, b in zip(x, y)]
            xn = rms(x, cfg.rms_eps, self.W[f"l{li}.ffn_norm"])
            f = self.ffn(li, xn)
            x = [a + b for a, b in zip(x, f)]
        xn = rms(x, cfg.rms_eps, self.W["final_norm"])
        return matvec(self.W["lm_head"], xn)


def _prefill_both(cfg, cache, naive, kvdt):
    for li in range(cfg.n_layers):
        k, v = gen.kv_prefill_bf16(cfg, li)
        for t in range(cfg.prefill):
            kf = [[bf(b) for b in k[t, g]] for g in range(cfg.n_kv_heads)]
            vf = [[bf(b) for b in v[t, g]] for g in range(cfg.n_kv_heads)]
            cache.store(li, t, np.array(kf), np.array(vf))
            naive.K[li][t] = [cache_round(kf[g], kvdt, naive.scales[li, g, 0] if naive.scales is not None else 1.0) for g in range(cfg.n_kv_heads)]
            naive.V[li][t] = [cache_round(vf[g], kvdt, naive.scales[li, g, 1] if naive.scales is not None else 1.0) for g in range(cfg.n_kv_heads)]


TINY_DENSE = DecodeConfig(name="naive_dense", n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2,
                          head_dim=8, ffn=48, vocab=37, prefill=5, n_decode=4, weight_sigma=0.3)
TINY_MOE = DecodeConfig(name="naive_moe", n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=1,
                        head_dim=8, ffn=0, vocab=29, n_experts=6, top_k=2, n_shared=1,
                        moe_ffn=32, prefill=3, n_decode=3, weight_sigma=0.3, lm_dtype="fp8")


def _run(cfg, kv_dtype="bf16", lm_fp8=False, gains="ones", windows=()):
    cfg = cfg.with_(kv_dtype=kv_dtype, norm_gains=gains, layer_window=tuple(windows))
    T = gen.dense_weights(cfg)
    if gains == "random":
        # three distinct non-unit gain vectors per layer plus the final one
        norms = [T[f"l{li}.{n}"] for li in range(cfg.n_layers) for n in ("attn_norm", "ffn_norm")]
        norms.append(T["final_norm"])
        for i, a in enumerate(norms):
            assert np.all(a != 0x3F80) or np.mean(a == 0x3F80) < 0.2
            for b in norms[i + 1:]:
                assert not np.array_equal(a, b)
    experts = (lambda l, e, w: gen.expert_mxfp4(cfg, l, e, w)) if cfg.is_moe else None
    lm = quantize_fp8_rows(T["lm_head"]) if lm_fp8 else None
    model = OracleModel(cfg, T, experts=experts, lm_fp8=lm)
    cache = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim, kv_dtype)
    naive = Naive(cfg, T, experts=experts, lm=lm)
    if kv_dtype == "fp8":
        sc = np.array([0.125, 0.25, 0.5, 0.0625], dtype=np.float32)
        cache.scales = np.stack([np.stack([sc[(l + g) % 4 : (l + g) % 4 + 1].repeat(2)
                                           for g in range(cfg.n_kv_heads)]) for l in range(cfg.n_layers)])
        cache.scales[:, :, 1] *= 2
        naive.scales = cache.scales
    _prefill_both(cfg, cache, naive, kv_dtype)
    toks = gen.prompt_tokens(cfg, cfg.n_decode)
    for j, tok in enumerate(toks):
        pos = cfg.prefill + j
        a = model.step(cache, int(tok), pos)
        b = np.array(naive.step(int(tok), pos))
        assert np.allclose(a, b, rtol=1e-9, atol=1e-9), (j, np.abs(a - b).max())


def test_naive_dense_bf16_kv():
    _run(TINY_DENSE)


def test_naive_dense_fp8_kv():
    _run(TINY_DENSE, kv_dtype="fp8")


def test_naive_dense_fp8_lm_head():
    _run(TINY_DENSE, lm_fp8=True)


def test_naive_moe():
    _run(TINY_MOE, lm_fp8=True)


def test_naive_dense_random_gains():
    _run(TINY_DENSE, gains="random")


def test_naive_dense_random_gains_fp8_kv():
    _run(TINY_DENSE, kv_dtype="fp8", gains="random")


def test_naive_moe_random_gains():
    _run(TINY_MOE, lm_fp8=True, gains="random")


@pytest.mark.parametrize("windows", [(3, 0), (1, 6), (2, 2)])
def test_naive_sliding_window(windows):
    """Sliding-window layers (the Muse Spark Open article, section on how
    the model is split): the brute-force loops attend the last W positions."""
    _run(TINY_DENSE, windows=windows)


def test_naive_sliding_window_moe_fp8_kv():
    _run(TINY_MOE, kv_dtype="fp8", windows=(2, 0))


def _first_step(cfg, T):
    m = OracleModel(cfg, T)
    c = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    return m.step(c, 3, 0)


@pytest.mark.parametrize("swap", ["attn_ffn", "final_dropped"])
def test_gain_placement_matters(swap):
    """A planted mistake in the oracle's gain placement (attention and FFN
    norms exchanged, or the final gain dropped) moves the logits far beyond
    the parity tolerance, so the gain tests above can see it."""
    cfg = TINY_DENSE.with_(norm_gains="random")
    T = gen.dense_weights(cfg)
    ref = _first_step(cfg, T)
    U = dict(T)
    if swap == "attn_ffn":
        for li in range(cfg.n_layers):
            U[f"l{li}.attn_norm"], U[f"l{li}.ffn_norm"] = T[f"l{li}.ffn_norm"], T[f"l{li}.attn_norm"]
    else:
        U["final_norm"] = gen.ones_bf16(T["final_norm"].shape)
    bad = _first_step(cfg, U)
    assert np.max(np.abs(bad - ref)) > 5e-2 * np.max(np.abs(ref))


def test_float32_mode_agrees_with_float64():
    cfg = TINY_DENSE.with_(hidden=64, ffn=128, head_dim=16, prefill=20, n_decode=6)
    T = gen.dense_weights(cfg)
    out = {}
    for dt in (np.float64, np.float32):
        m = OracleModel(cfg, T, dtype=dt)
        c = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
        for li in range(cfg.n_layers):
            k, v = gen.kv_prefill_bf16(cfg, li)
            c.k[li][:cfg.prefill] = k
            c.v[li][:cfg.prefill] = v
        out[dt] = [m.step(c, 3 + j, cfg.prefill + j) for j in range(cfg.n_decode)]
    for a, b in zip(out[np.float64], out[np.float32]):
        rel = np.linalg.norm(a - b) / np.linalg.norm(a)
        assert rel < 1e-5


def test_verify_is_steps_in_sequence():
    cfg = TINY_DENSE
    T = gen.dense_weights(cfg)
    m = OracleModel(cfg, T)
    c1 = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    c2 = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    toks = [3, 1, 4, 1]
    a = m.verify(c1, toks, 2)
    b = np.stack([m.step(c2, t, 2 + j) for j, t in enumerate(toks)])
    assert np.array_equal(a, b)
    assert np.array_equal(c1.k[1], c2.k[1])
