"""Plain CPU forward step of a batch-1 decoder (float64 by default).

TEST INFRASTRUCTURE: see the package docstring.

What one decode step computes, as the decode-speed pages describe it: every
generated token is a chain of matrix-vector products over all active weights
(Kog article "Real-time LLM inference on standard GPUs: 3k tokens/s per
request", section on memory bandwidth as the bottleneck); a routed MoE layer
reads only the top-8 of 512 experts plus one shared expert, and a verify pass
runs the target model over a 4-token window (163.com Ling-3.0-flash article,
sections "model and baseline configuration" and "optimisation 3: MTP
speculative decoding with NEXTN"); the LM head may be stored as FP8 with a
per-row scale (same article, "optimisation 2"); the KV cache may be FP8 with a
per-head scale (wmrh.cn Kimi-K3 report, test environment and warnings).

Where the pages are silent the plainest reading is taken:
  * RMSNorm y = x / sqrt(mean(x^2) + eps) * g, eps = 1e-6;
  * RoPE rotates pairs (i, i + d/2) by pos * theta^(-2i/d);
  * query head h reads KV head floor(h * Hkv / Hq);
  * attention is causal softmax(q.k / sqrt(d)) over positions [0, pos],
    including the K/V just written at pos, read back in cache precision;
  * a sliding-window layer of window W ("Muse Spark Open" article, section
    on how the model is split: layers attending over the last 2,048 tokens)
    attends the W most recent positions, [max(0, pos - W + 1), pos], its
    own included;
  * SwiGLU: W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + e^-z);
  * MoE: p = softmax(W_router x); the top-k of p (lower index wins ties)
    are renormalised to sum to 1; the shared expert is added with weight 1;
  * logits = W_lm rmsnorm(x); argmax takes the lowest index on ties;
  * no biases; untied embedding and LM head.
Activations stay in the working precision (float64 unless asked otherwise);
only the KV cache is stored narrow.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

from . import codecs

# ---------------------------------------------------------------------------
# Building blocks
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate each head of x [n_heads][d] at position `pos` (half-split pairs).

    Angles are formed in float64 and, in the float32 working mode, their
    cosine and sine are rounded to float32, as a table kept in float32 would
    hold them.
    """
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    if x.dtype == np.float32:
        c, s = c.astype(np.float32), s.astype(np.float32)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def softmax(z: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Single-query grouped attention.

    q [Hq][d]; k, v [T][Hkv][d] (positions 0..T-1, all visible).
    Returns o [Hq][d]: o_h = sum_t softmax_t(q_h . k_t / sqrt(d)) v_t using
    KV head floor(h * Hkv / Hq).
    """
    Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.empty_like(q)
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = (k[:, g, :] @ q[h]) / np.sqrt(d)
        p = softmax(s)
        out[h] = p @ v[:, g, :]
    return out


def window_start(pos: int, window: int) -> int:
    """First position a token at `pos` attends in a layer of window W
    (0 = global): the W most recent positions, its own included."""
    return max(0, pos - window + 1) if window > 0 else 0


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    return wd @ (silu(wg @ x) * (wu @ x))


def topk_lower_index(values: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest values; equal values go to the lower index."""
    order = np.lexsort((np.arange(values.size), -values))
    return order[:k]


def argmax_lower_index(values: np.ndarray) -> int:
    return int(topk_lower_index(values, 1)[0])


def route(router_logits: np.ndarray, k: int):
    """Softmax router, top-k, renormalised weights.

    The selection is decided on binary32 logits (the precision the GPU
    holds them in); softmax is monotone, so the top-k of p is the top-k of
    the logits.  Returns (indices int64 [k], weights [k]).
    """
    sel = topk_lower_index(router_logits.astype(np.float32).astype(np.float64), k)
    p = softmax(router_logits)
    w = p[sel] / np.sum(p[sel])
    return sel, w


def quantize_fp8_rows(w_bf16: np.ndarray):
    """Online FP8 quantisation of a BF16 matrix, one fp32 scale per row.

    163.com Ling-3.0-flash article, "optimisation 2: online FP8 LM head
    quantisation": the BF16 LM head is converted to FP8 when it is built,
    halving its reads.  Per row: amax = max |w| (exact in binary32),
    scale = amax / 448 in binary32 (1.0 for an all-zero row), and
    code = E4M3FN(w / scale) with the division in binary32, nearest-even,
    saturating.  Returns (codes u8 [rows][cols], scales f32 [rows]).
    """
    w = codecs.bf16_to_f64(w_bf16).astype(np.float32)
    amax = np.max(np.abs(w), axis=1)
    scale = (amax / np.float32(codecs.FP8_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        y = (w / scale[:, None]).astype(np.float32)
    return codecs.f32_to_fp8e4m3(y), scale


def dequant_fp8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return codecs.fp8e4m3_to_f64(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def lm_head_logits(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    return w @ x


# ---------------------------------------------------------------------------
# KV cache (logical; page placement is a GPU-side layout detail)
# ---------------------------------------------------------------------------


@dataclass
class OracleCache:
    """K/V of every layer by position, held in the cache's storage format.

    kv_dtype "bf16": uint16 BF16 bits; "fp8": uint8 E4M3FN codes with one
    binary32 scale per (layer, KV head, K or V), value = decode(code) *
    scale.
    """
    n_layers: int
    max_pos: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str = "bf16"
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)
    scales: Optional[np.ndarray] = None   # float32 [L][Hkv][2]

    def __post_init__(self):
        dt = np.uint16 if self.kv_dtype == "bf16" else np.uint8
        shp = (self.max_pos, self.n_kv_heads, self.head_dim)
        if not self.k:
            self.k = [np.zeros(shp, dtype=dt) for _ in range(self.n_layers)]
            self.v = [np.zeros(shp, dtype=dt) for _ in range(self.n_layers)]
        if self.kv_dtype == "fp8" and self.scales is None:
            self.scales = np.ones((self.n_layers, self.n_kv_heads, 2), dtype=np.float32)

    def store(self, layer: int, pos: int, k: np.ndarray, v: np.ndarray) -> None:
        """Write K/V rows [Hkv][d] at `pos` in cache precision.

        BF16: value -> binary32 -> BF16 nearest-even.  FP8: binary32(value)
        / scale in binary32, then E4M3FN nearest-even with saturation.
        """
        if self.kv_dtype == "bf16":
            self.k[layer][pos] = codecs.round_to_bf16(k)
            self.v[layer][pos] = codecs.round_to_bf16(v)
        else:
            for which, src, dst in ((0, k, self.k[layer]), (1, v, self.v[layer])):
                sc = self.scales[layer, :, which].astype(np.float32)[:, None]
                y = (np.asarray(src, dtype=np.float64).astype(np.float32) / sc).astype(np.float32)
                dst[pos] = codecs.f32_to_fp8e4m3(y)

    def prefill_f32(self, layer: int, pos0: int, k: np.ndarray, v: np.ndarray) -> None:
        """Store float32 K/V rows [n][Hkv][d] at positions pos0 .. pos0+n-1,
        rounded to the cache format as `store` does (bulk form)."""
        n = k.shape[0]
        if self.kv_dtype == "bf16":
            self.k[layer][pos0:pos0 + n] = codecs.f32_to_bf16(np.asarray(k, dtype=np.float32))
            self.v[layer][pos0:pos0 + n] = codecs.f32_to_bf16(np.asarray(v, dtype=np.float32))
            return
        for which, src, dst in ((0, k, self.k[layer]), (1, v, self.v[layer])):
            sc = self.scales[layer, :, which].astype(np.float32)[None, :, None]
            y = (np.asarray(src, dtype=np.float32) / sc).astype(np.float32)
            dst[pos0:pos0 + n] = codecs.f32_to_fp8e4m3_bulk(y)

    def read(self, layer: int, upto: int, dtype=np.float64):
        """Dequantised K, V for positions [0, upto), [T][Hkv][d]."""
        if self.kv_dtype == "bf16":
            k = codecs.bf16_to_f64(self.k[layer][:upto])
            v = codecs.bf16_to_f64(self.v[layer][:upto])
        else:
            sk = self.scales[layer, :, 0].astype(np.float64)[:, None]
            sv = self.scales[layer, :, 1].astype(np.float64)[:, None]
            k = codecs.fp8e4m3_to_f64_bulk(self.k[layer][:upto], sk)
            v = codecs.fp8e4m3_to_f64_bulk(self.v[layer][:upto], sv)
        return k.astype(dtype, copy=False), v.astype(dtype, copy=False)


# ---------------------------------------------------------------------------
# Model
# ---------------------------------------------------------------------------


class OracleModel:
    """A decoder given by its stored tensors.

    tensors: dict of BF16-bit arrays, keys ``embed``, ``final_norm``,
    ``lm_head`` and ``l{i}.{attn_norm,wq,wk,wv,wo,ffn_norm}`` plus either
    ``l{i}.{w_gate,w_up,w_down}`` (dense) or ``l{i}.w_router`` (MoE).
    experts: for MoE, a callable (layer, expert, which) -> (codes, scales) of
    an MXFP4 matrix, which in {"gate_up", "down"}; expert index n_experts is
    the shared expert.
    lm_fp8: optional (codes, scales) replacing the BF16 LM head.
    """

    def __init__(self, cfg, tensors: dict, experts: Optional[Callable] = None,
                 lm_fp8=None, dtype=np.float64, cache_weights: bool = True, cache_experts: bool = True):
        self.cfg = cfg
        self.t = tensors
        self.experts = experts
        self.lm_fp8 = lm_fp8
        self.dtype = dtype
        self.cache_weights = cache_weights
        self.cache_experts = cache_experts
        self._w = {}
        self.last_routing = []   # per layer: (indices, weights, router logits)

    # -- weights -----------------------------------------------------------
    def w(self, name: str) -> np.ndarray:
        if name in self._w:
            return self._w[name]
        if name == "lm_head" and self.lm_fp8 is not None:
            m = dequant_fp8_rows(*self.lm_fp8)
        else:
            m = codecs.bf16_to_f64(self.t[name])
        m = m.astype(self.dtype)
        if self.cache_weights:
            self._w[name] = m
        return m

    def expert(self, layer: int, e: int):
        key = f"l{layer}.expert{e}"
        if key in self._w:
            return self._w[key]
        gu = codecs.mxfp4_to_f64_bulk(*self.experts(layer, e, "gate_up")).astype(self.dtype, copy=False)
        dn = codecs.mxfp4_to_f64_bulk(*self.experts(layer, e, "down")).astype(self.dtype, copy=False)
        mf = self.cfg.moe_ffn
        out = (gu[:mf], gu[mf:], dn)
        if self.cache_weights and self.cache_experts:
            self._w[key] = out
        return out

    def window(self, li: int) -> int:
        w = getattr(self.cfg, "layer_window", ())
        return int(w[li]) if w else 0

    # -- one layer ---------------------------------------------------------
    def _ffn(self, li: int, xn: np.ndarray) -> np.ndarray:
        cfg = self.cfg
        if not cfg.is_moe:
            return swiglu(xn, self.w(f"l{li}.w_gate"), self.w(f"l{li}.w_up"),
                          self.w(f"l{li}.w_down"))
        r = self.w(f"l{li}.w_router") @ xn
        sel, wts = route(r, cfg.top_k)
        self.last_routing.append((sel, wts, r))
        y = np.zeros_like(xn)
        for e, we in zip(sel, wts):
            g, u, dn = self.expert(li, int(e))
            y = y + we * swiglu(xn, g, u, dn)
        for s in range(cfg.n_shared):
            g, u, dn = self.expert(li, cfg.n_experts + s)
            y = y + swiglu(xn, g, u, dn)
        return y

    def step(self, cache: OracleCache, token: int, pos: int) -> np.ndarray:
        """One decode step: embed `token`, write K/V at `pos`, return logits."""
        cfg = self.cfg
        dt = self.dtype
        eps = cfg.rms_eps
        d = cfg.head_dim
        self.last_routing = []
        x = codecs.bf16_to_f64(self.t["embed"][token]).astype(dt)
        for li in range(cfg.n_layers):
            xn = rmsnorm(x, self.w(f"l{li}.attn_norm"), eps)
            q = (self.w(f"l{li}.wq") @ xn).reshape(cfg.n_q_heads, d)
            k = (self.w(f"l{li}.wk") @ xn).reshape(cfg.n_kv_heads, d)
            v = (self.w(f"l{li}.wv") @ xn).reshape(cfg.n_kv_heads, d)
            q = rope(q, pos, cfg.rope_theta)
            k = rope(k, pos, cfg.rope_theta)
            cache.store(li, pos, k, v)
            kc, vc = cache.read(li, pos + 1, dt)
            lo = window_start(pos, self.window(li))
            o = attention(q, kc[lo:], vc[lo:]).reshape(-1)
            x = x + self.w(f"l{li}.wo") @ o
            xn = rmsnorm(x, self.w(f"l{li}.ffn_norm"), eps)
            x = x + self._ffn(li, xn)
        xn = rmsnorm(x, self.w("final_norm"), eps)
        self.last_hidden = xn
        return self.w("lm_head") @ xn

    def verify(self, cache: OracleCache, tokens, pos: int) -> np.ndarray:
        """Verify window: token j at position pos + j sees [0, pos + j] (in a
        sliding-window layer the last W of them), the window's earlier
        tokens included.  Returns logits [k][vocab]."""
        return np.stack([self.step(cache, int(t), pos + j) for j, t in enumerate(tokens)])


# ---------------------------------------------------------------------------
# Speculative round
# ---------------------------------------------------------------------------


def spec_round(target, tcache, draft, dcache, token: int, pos: int, k: int):
    """One greedy speculative round (163.com Ling-3.0-flash article,
    optimisation 3: a draft proposes tokens, the target checks the 4-token
    window in one pass and keeps the prefix it agrees with).

    The draft (any model with .step(cache, token, pos) -> logits) runs k
    greedy steps from `token` at pos .. pos + k - 1; the window is `token`
    and its first k - 1 proposals (the k-th step only extends the draft's
    cache).  The target verifies the window at pos; am[j] is its argmax after
    window[j].  Draft token j + 1 is accepted while am[j] == window[j + 1];
    with m accepted the round emits am[0 .. m] and the next round starts from
    am[m] at pos + m + 1.  Returns (emitted, next_pos, next_token, window,
    target window logits)."""
    window = [int(token)]
    t = int(token)
    for s in range(k):
        t = argmax_lower_index(draft.step(dcache, t, pos + s))
        window.append(t)
    logits = target.verify(tcache, window[:k], pos)
    am = [argmax_lower_index(v) for v in logits]
    m = 0
    while m < k - 1 and am[m] == window[m + 1]:
        m += 1
    return am[:m + 1], pos + m + 1, am[m], window, logits

