"""Seeded synthetic inputs shared by the oracle and the GPU path.

Every array here is a pure function of (seed, tensor name, shape).  The module
draws random numbers and lays them out; it holds none of the decode step's
arithmetic (no rounding to cache formats, no quantisation, no normalisation).

Seeds (root seed 0 for weights):
  * weights: ``SeedSequence([0, crc32(name)])``, PCG64, float32 normal x sigma,
    stored as BF16 by dropping the low 16 bits of the float32 sample
    (truncation: a way to draw BF16 numbers, not the decode path's rounding);
  * prompt token ids: seed 1, uniform over [0, vocab);
  * K/V prefill: seed 2, N(0, 1) per (layer, K or V), BF16 by truncation;
    for a float32 prefill of hundreds of thousands of positions (the
    long-context FP8 cache), N(0, 1) drawn on the GPU by torch's generator,
    seeded per (seed 2, layer, K or V, block of KV_BLOCK positions);
  * non-unit RMSNorm gains (the "random" gain option): per norm tensor,
    ``SeedSequence([5, crc32(name)])``, float32 1 + 0.1 N(0, 1), BF16 by
    truncation, so every norm of every layer gets its own vector;
  * page-table shuffle: seed 3, a uniform permutation of the physical pages;
  * LM-head input vectors: seed 4, float32 N(0, 1);
  * MXFP4 expert codes and scales: a counter-based integer hash (SplitMix64,
    Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
    OOPSLA 2014) of (tensor id, byte index), so that any expert can be drawn
    on its own without drawing the ones before it.
"""
from __future__ import annotations

import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import DecodeConfig

ROOT_SEED = 0
PROMPT_SEED = 1
KV_SEED = 2
PAGE_SEED = 3
XVEC_SEED = 4
GAIN_SEED = 5

BF16_ONE = np.uint16(0x3F80)

_POOL = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=8)
    return _POOL


def tensor_id(name: str) -> int:
    return zlib.crc32(name.encode("utf-8"))


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(words))))


def _f32_to_bf16_bits_trunc(x: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def normal_bf16(name: str, shape, sigma: float, seed: int = ROOT_SEED) -> np.ndarray:
    """BF16 bit patterns of sigma * N(0, 1) draws for tensor `name`."""
    rng = _rng(seed, tensor_id(name))
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    x *= np.float32(sigma)
    return _f32_to_bf16_bits_trunc(x).reshape(shape)


def ones_bf16(shape) -> np.ndarray:
    return np.full(shape, BF16_ONE, dtype=np.uint16)


def gain_bf16(name: str, shape, spread: float = 0.1) -> np.ndarray:
    """BF16 bit patterns of 1 + spread * N(0, 1) draws for norm `name`."""
    rng = _rng(GAIN_SEED, tensor_id(name))
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    x = np.float32(1.0) + np.float32(spread) * x
    return _f32_to_bf16_bits_trunc(x).reshape(shape)


# ---------------------------------------------------------------------------
# Weights
# ---------------------------------------------------------------------------

def layer_tensor_shapes(cfg: DecodeConfig) -> dict:
    """Shapes of one decoder layer's BF16 tensors, [out][in] row-major."""
    H, d = cfg.hidden, cfg.head_dim
    s = {
        "attn_norm": (H,),
        "wq": (cfg.n_q_heads * d, H),
        "wk": (cfg.n_kv_heads * d, H),
        "wv": (cfg.n_kv_heads * d, H),
        "wo": (H, cfg.n_q_heads * d),
        "ffn_norm": (H,),
    }
    if cfg.is_moe:
        s["w_router"] = (cfg.n_experts, H)
    else:
        s["w_gate"] = (cfg.ffn, H)
        s["w_up"] = (cfg.ffn, H)
        s["w_down"] = (H, cfg.ffn)
    return s


def dense_weights(cfg: DecodeConfig, with_lm_head: bool = True) -> dict:
    """All BF16 tensors of a model, generated in parallel (one stream each).

    Keys: ``embed``, ``final_norm``, ``lm_head`` and ``l{i}.{tensor}``.  MoE
    expert tensors are not included (see ``expert_mxfp4``).  Norm gains are
    1.0 unless ``cfg.norm_gains == "random"``.
    """
    jobs = {}
    V, H = cfg.vocab, cfg.hidden
    sig = cfg.weight_sigma
    if cfg.n_layers > 0:
        jobs["embed"] = ("normal", (V, H))
        jobs["final_norm"] = ("ones", (H,))
    if with_lm_head:
        jobs["lm_head"] = ("normal", (V, H))
    for li in range(cfg.n_layers):
        for t, shp in layer_tensor_shapes(cfg).items():
            kind = "ones" if t.endswith("norm") else "normal"
            jobs[f"l{li}.{t}"] = (kind, shp)

    def run(item):
        name, (kind, shp) = item
        if kind == "ones":
            if cfg.norm_gains == "random":
                return name, gain_bf16(f"{cfg.name}.{name}", shp)
            return name, ones_bf16(shp)
        return name, normal_bf16(f"{cfg.name}.{name}", shp, sig)

    return dict(_pool().map(run, jobs.items()))


def lm_head_bf16(cfg: DecodeConfig) -> np.ndarray:
    return normal_bf16(f"{cfg.name}.lm_head", (cfg.vocab, cfg.hidden), cfg.weight_sigma)


def lm_head_inputs(cfg: DecodeConfig, k: int) -> np.ndarray:
    """k hidden vectors ~ N(0, 1), float32, shape [k][hidden]."""
    return _rng(XVEC_SEED, k).standard_normal((k, cfg.hidden), dtype=np.float32)


# ---------------------------------------------------------------------------
# Tokens, KV prefill, page table
# ---------------------------------------------------------------------------

def prompt_tokens(cfg: DecodeConfig, n: int) -> np.ndarray:
    return _rng(PROMPT_SEED).integers(0, cfg.vocab, size=n, dtype=np.int64).astype(np.int32)


def kv_prefill_bf16(cfg: DecodeConfig, layer: int) -> tuple:
    """Logical K and V of positions [0, prefill) for one layer.

    Returns two BF16-bit arrays of shape [prefill][n_kv_heads][head_dim]
    drawn from N(0, 1).  Where they sit in a paged pool is the caller's
    business.
    """
    shp = (cfg.prefill, cfg.n_kv_heads, cfg.head_dim)
    out = []
    for kv in (0, 1):
        x = _rng(KV_SEED, layer, kv).standard_normal(int(np.prod(shp)), dtype=np.float32)
        out.append(_f32_to_bf16_bits_trunc(x).reshape(shp))
    return out[0], out[1]


KV_BLOCK = 8192


def _block_seed(*words: int) -> int:
    return int(np.random.SeedSequence(list(words)).generate_state(1, np.uint64)[0] & np.uint64(2**63 - 1))


def kv_prefill_f32_device(cfg: DecodeConfig, layer: int, kv: int, start: int, n: int, device):
    """float32 N(0, 1) rows [n][n_kv_heads][head_dim] of K (kv = 0) or V
    (kv = 1) for positions [start, start + n) of `layer`, as a torch tensor
    on `device`.

    Positions are drawn in blocks of KV_BLOCK, each from torch's generator on
    that device seeded with (KV_SEED, layer, kv, block), so any range can be
    drawn without the ones before it and both sides of a comparison draw the
    same numbers.
    """
    import torch
    shp = (cfg.n_kv_heads, cfg.head_dim)
    out = torch.empty((n, *shp), dtype=torch.float32, device=device)
    if n == 0:
        return out
    for b in range(start // KV_BLOCK, (start + n - 1) // KV_BLOCK + 1):
        g = torch.Generator(device=device)
        g.manual_seed(_block_seed(KV_SEED, layer, kv, b))
        blk = torch.randn((KV_BLOCK, *shp), generator=g, device=device, dtype=torch.float32)
        lo, hi = max(start, b * KV_BLOCK), min(start + n, (b + 1) * KV_BLOCK)
        out[lo - start:hi - start] = blk[lo - b * KV_BLOCK:hi - b * KV_BLOCK]
    return out


def page_table(cfg: DecodeConfig, shuffled: bool | None = None) -> np.ndarray:
    """Logical page -> physical page, int32 [n_pages]."""
    if shuffled is None:
        shuffled = cfg.shuffled_pages
    n = cfg.n_pages
    if not shuffled:
        return np.arange(n, dtype=np.int32)
    return _rng(PAGE_SEED, n).permutation(n).astype(np.int32)


def batch_page_table(cfg: DecodeConfig, n_seqs: int, shuffled: bool | None = None) -> np.ndarray:
    """Page tables of n_seqs sequences sharing one pool, int32
    [n_seqs][n_pages]: disjoint physical pages (a permutation of
    n_seqs * n_pages when shuffled, else consecutive blocks)."""
    if shuffled is None:
        shuffled = cfg.shuffled_pages
    n = cfg.n_pages
    phys = np.arange(n_seqs * n, dtype=np.int32)
    if shuffled:
        phys = _rng(PAGE_SEED + 1, n_seqs * n).permutation(n_seqs * n).astype(np.int32)
    return phys.reshape(n_seqs, n)


# ---------------------------------------------------------------------------
# Counter-based draws (MXFP4 experts)
# ---------------------------------------------------------------------------

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)


def splitmix64(counter: np.ndarray) -> np.ndarray:
    """SplitMix64 output for state value `counter` (already advanced).

    The generator's n-th output from seed s is ``splitmix64(s + n * gamma)``
    with gamma = 0x9E3779B97F4A7C15 (n counted from 1).
    """
    z = np.asarray(counter, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def hash_stream(stream: int, index: np.ndarray) -> np.ndarray:
    """64-bit hash of (stream, index): SplitMix64 state = stream*2^40 + index + 1, times gamma."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = (np.uint64(stream) << np.uint64(40)) + idx + np.uint64(1)
        state = state * GOLDEN_GAMMA
    return splitmix64(state)


def expert_mxfp4(cfg: DecodeConfig, layer: int, expert: int, which: str) -> tuple:
    """Codes and E8M0 scales of one expert matrix.

    which: "gate_up" -> [2*moe_ffn][hidden] (gate rows then up rows),
           "down"    -> [hidden][moe_ffn].
    Expert index ``cfg.n_experts`` is the shared expert.
    Codes: every nibble uniform over the 16 E2M1 codes, two per byte.
    Scales: E8M0 bytes uniform over {120, 121, 122}, i.e. 2^-7 .. 2^-5.
    Returns (codes u8 [rows][cols/2], scales u8 [rows][cols/32]).
    """
    if which == "gate_up":
        rows, cols = 2 * cfg.moe_ffn, cfg.hidden
        kind = 0
    else:
        rows, cols = cfg.hidden, cfg.moe_ffn
        kind = 1
    stream = ((layer * (cfg.n_experts + 1) + expert) * 2 + kind) * 2
    nb = rows * cols // 2
    ns = rows * cols // 32
    # one 64-bit hash yields 8 code bytes / 8 scale draws
    hc = hash_stream(stream, np.arange(-(-nb // 8), dtype=np.uint64))
    codes = hc.view(np.uint8)[:nb].reshape(rows, cols // 2).copy()
    hs = hash_stream(stream + 1, np.arange(-(-ns // 8), dtype=np.uint64))
    sb = hs.view(np.uint8)[:ns].astype(np.uint16)
    scales = (np.uint16(120) + (sb * np.uint16(3) >> np.uint16(8))).astype(np.uint8)
    return codes, scales.reshape(rows, cols // 32)


# torch forms of the counter hash, so that experts of full-size models can be
# drawn where they are used (on the GPU).  Same bits as the numpy functions:
# int64 arithmetic wraps modulo 2^64 like uint64, and right shifts are made
# logical with a mask.

def _i64(u: int) -> int:
    return u - (1 << 64) if u >= 1 << 63 else u


def _lsr(z, k: int):
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64_torch(state):
    z = state.clone()
    z ^= _lsr(z, 30)
    z *= _i64(0xBF58476D1CE4E5B9)
    z ^= _lsr(z, 27)
    z *= _i64(0x94D049BB133111EB)
    z ^= _lsr(z, 31)
    return z


def hash_stream_torch(stream: int, start: int, n: int, device):
    """hash_stream(stream, start .. start+n-1) as an int64 torch tensor."""
    import torch
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    state = (idx + ((stream << 40) + 1)) * _i64(int(GOLDEN_GAMMA))
    return splitmix64_torch(state)


def expert_mxfp4_torch(cfg: DecodeConfig, layer: int, expert: int, which: str, codes_out, scales_out) -> None:
    """expert_mxfp4 written into torch uint8 tensors (any device) of shapes
    [rows][cols/2] and [rows][cols/32]."""
    import torch
    if which == "gate_up":
        rows, cols, kind = 2 * cfg.moe_ffn, cfg.hidden, 0
    else:
        rows, cols, kind = cfg.hidden, cfg.moe_ffn, 1
    stream = ((layer * (cfg.n_experts + 1) + expert) * 2 + kind) * 2
    nb = rows * cols // 2
    ns = rows * cols // 32
    dev = codes_out.device
    hc = hash_stream_torch(stream, 0, -(-nb // 8), dev)
    codes_out.view(-1).copy_(hc.view(torch.uint8)[:nb])
    hs = hash_stream_torch(stream + 1, 0, -(-ns // 8), dev)
    sb = hs.view(torch.uint8)[:ns].to(torch.int32)
    scales_out.view(-1).copy_((120 + ((sb * 3) >> 8)).to(torch.uint8))


def experts_mxfp4_torch(cfg: DecodeConfig, layer: int, experts, which: str, codes_out, scales_out,
                        chunk: int = 64) -> None:
    """expert_mxfp4 of every expert id in `experts`, written into stacked
    torch uint8 tensors codes_out [n][rows][cols/2], scales_out [n][rows][cols/32]."""
    import torch
    if which == "gate_up":
        rows, cols, kind = 2 * cfg.moe_ffn, cfg.hidden, 0
    else:
        rows, cols, kind = cfg.hidden, cfg.moe_ffn, 1
    nb = rows * cols // 2
    ns = rows * cols // 32
    dev = codes_out.device
    ids = list(experts)
    gamma = _i64(int(GOLDEN_GAMMA))
    for i0 in range(0, len(ids), chunk):
        part = ids[i0:i0 + chunk]
        streams = torch.tensor([((layer * (cfg.n_experts + 1) + e) * 2 + kind) * 2 for e in part],
                               dtype=torch.int64, device=dev)[:, None]
        for off, n, out in ((0, nb, codes_out), (1, ns, scales_out)):
            idx = torch.arange(-(-n // 8), dtype=torch.int64, device=dev)[None, :]
            h = splitmix64_torch((((streams + off) << 40) + idx + 1) * gamma)
            b = h.view(torch.uint8).view(len(part), -1)[:, :n]
            if off == 1:
                b = (120 + ((b.to(torch.int32) * 3) >> 8)).to(torch.uint8)
            out[i0:i0 + len(part)].view(len(part), -1).copy_(b)
