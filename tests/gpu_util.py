"""Shared helpers of the GPU parity tests: build the same synthetic model on
the device (through the C-ABI) and in the CPU oracle, and compare."""
from __future__ import annotations

import sys

import numpy as np

from oracle import OracleCache, OracleModel
from synth import gen

LOGIT_MAX_ABS = 2e-2
LOGIT_REL_L2 = 5e-3          # BF16 / FP8 weights
LOGIT_REL_L2_MXFP4 = 1e-2
ARGMAX_MARGIN = 1e-2


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def compare_logits(gpu: np.ndarray, ref: np.ndarray, rel_tol=LOGIT_REL_L2, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU logits"
    max_abs = float(np.max(np.abs(gpu - ref)))
    rel = float(np.linalg.norm(gpu - ref) / np.linalg.norm(ref))
    assert max_abs <= LOGIT_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {LOGIT_MAX_ABS}"
    assert rel <= rel_tol, f"{what}: rel L2 {rel:.3e} > {rel_tol}"
    return max_abs, rel


def top2_margin(ref: np.ndarray) -> float:
    s = np.sort(ref)
    return float(s[-1] - s[-2])


def lowest_argmax(v: np.ndarray) -> int:
    m = np.max(v)
    return int(np.flatnonzero(v == m)[0])


def check_argmax(gpu_idx: int, gpu_logits: np.ndarray, ref: np.ndarray, what=""):
    # the GPU's index is exactly the lowest argmax of the GPU's own logits
    assert gpu_idx == lowest_argmax(gpu_logits), f"{what}: argmax {gpu_idx} not the lowest max of its logits"
    if top2_margin(ref) > ARGMAX_MARGIN:
        assert gpu_idx == lowest_argmax(ref), f"{what}: argmax {gpu_idx} != oracle {lowest_argmax(ref)}"
        return True
    return False


FP8_MAX = 448.0


def fp8_kv_scales(cfg, block: int = 1 << 16):
    """Per (layer, KV head, K or V) power-of-two scale 2^ceil(log2(amax / 448))
    over the float32 prefill samples (float32 [L][Hkv][2])."""
    import torch
    sc = np.ones((cfg.n_layers, cfg.n_kv_heads, 2), dtype=np.float32)
    if not cfg.prefill:
        return sc
    for li in range(cfg.n_layers):
        for kv in (0, 1):
            am = torch.zeros(cfg.n_kv_heads, dtype=torch.float32, device="cuda")
            for p0 in range(0, cfg.prefill, block):
                n = min(block, cfg.prefill - p0)
                x = gen.kv_prefill_f32_device(cfg, li, kv, p0, n, "cuda")
                am = torch.maximum(am, x.abs().amax(dim=(0, 2)))
            a = am.double().cpu().numpy()
            sc[li, :, kv] = np.exp2(np.ceil(np.log2(a / FP8_MAX))).astype(np.float32)
    return sc


def build_dense(cfg, shuffled=None, kv_dtype=None, kv_scales=None, k_max=None, host=None, block=1 << 16,
                prefill_lens=None):
    """(DeviceModel, OracleModel, OracleCache) with identical weights and prefill.

    BF16 caches take their prefill as BF16 draws placed directly in both
    caches.  FP8 caches take float32 draws (made on the GPU) that each side
    rounds into its own cache: the library through mbg_kv_write, the oracle
    through its codec.  prefill_lens (one length per sequence, each at most
    cfg.prefill) builds several sequences on disjoint pages; the third item
    is then a list of oracle caches, sequence b holding the first
    prefill_lens[b] prefill positions."""
    import torch
    from memory_bound_gemv_amd.device_model import DeviceModel
    kv_dtype = kv_dtype or cfg.kv_dtype
    host = host if host is not None else gen.dense_weights(cfg)
    lens = [cfg.prefill] if prefill_lens is None else list(prefill_lens)
    pt = gen.page_table(cfg, shuffled) if prefill_lens is None else gen.batch_page_table(cfg, len(lens), shuffled)
    if kv_dtype == "fp8" and kv_scales is None:
        kv_scales = fp8_kv_scales(cfg, block)
    dm = DeviceModel(cfg, host, pt, kv_dtype=kv_dtype, kv_scales=kv_scales, k_max=k_max)
    om = OracleModel(cfg, host)
    ocs = [OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim, kv_dtype) for _ in lens]
    for oc in ocs:
        if kv_dtype == "fp8":
            oc.scales = np.asarray(kv_scales, dtype=np.float32).reshape(cfg.n_layers, cfg.n_kv_heads, 2)
    if cfg.prefill:
        for li in range(cfg.n_layers):
            k, v = gen.kv_prefill_bf16(cfg, li)
            for b, (T, oc) in enumerate(zip(lens, ocs)):
                if kv_dtype == "bf16":
                    dm.prefill_bf16(li, k[:T], v[:T], seq=b)
                    oc.k[li][:T] = k[:T]
                    oc.v[li][:T] = v[:T]
                else:
                    for p0 in range(0, T, block):
                        n = min(block, T - p0)
                        kd = gen.kv_prefill_f32_device(cfg, li, 0, p0, n, "cuda")
                        vd = gen.kv_prefill_f32_device(cfg, li, 1, p0, n, "cuda")
                        dm.kv_write(li, p0, kd, vd, seq=b)
                        oc.prefill_f32(li, p0, kd.cpu().numpy(), vd.cpu().numpy())
                    torch.cuda.synchronize()
    oc = ocs[0] if prefill_lens is None else ocs
    dm.init()
    return dm, om, oc


def device_experts(cfg, device="cuda"):
    """Every layer's MXFP4 experts, drawn on the device by the counter hash."""
    import torch
    E, S, H, Mf = cfg.n_experts, cfg.n_shared, cfg.hidden, cfg.moe_ffn
    u8 = dict(dtype=torch.uint8, device=device)
    out = []
    for li in range(cfg.n_layers):
        d = dict(eg_codes=torch.empty((E, 2 * Mf, H // 2), **u8), eg_scales=torch.empty((E, 2 * Mf, H // 32), **u8),
                 ed_codes=torch.empty((E, H, Mf // 2), **u8), ed_scales=torch.empty((E, H, Mf // 32), **u8),
                 sg_codes=torch.empty((max(S, 1), 2 * Mf, H // 2), **u8),
                 sg_scales=torch.empty((max(S, 1), 2 * Mf, H // 32), **u8),
                 sd_codes=torch.empty((max(S, 1), H, Mf // 2), **u8),
                 sd_scales=torch.empty((max(S, 1), H, Mf // 32), **u8))
        gen.experts_mxfp4_torch(cfg, li, range(E), "gate_up", d["eg_codes"], d["eg_scales"])
        gen.experts_mxfp4_torch(cfg, li, range(E), "down", d["ed_codes"], d["ed_scales"])
        if S:
            gen.experts_mxfp4_torch(cfg, li, range(E, E + S), "gate_up", d["sg_codes"], d["sg_scales"])
            gen.experts_mxfp4_torch(cfg, li, range(E, E + S), "down", d["sd_codes"], d["sd_scales"])
        out.append(d)
    torch.cuda.synchronize()
    return out


def build_moe(cfg, shuffled=None, k_max=None, host=None, cache_experts=True, prefill_lens=None):
    """(DeviceModel, OracleModel, OracleCache) of a routed model: BF16
    attention/router weights, MXFP4 experts (drawn on the device for the
    library, regenerated per expert on the host for the oracle), FP8 LM head
    quantised from the same BF16 head by each side on its own (the library's
    mbg_quantize_fp8_rows, the oracle's quantize_fp8_rows)."""
    import torch
    from memory_bound_gemv_amd import _mbg as M
    from memory_bound_gemv_amd.device_model import DeviceModel
    from oracle import quantize_fp8_rows
    host = host if host is not None else gen.dense_weights(cfg)
    lens = [cfg.prefill] if prefill_lens is None else list(prefill_lens)
    pt = gen.page_table(cfg, shuffled) if prefill_lens is None else gen.batch_page_table(cfg, len(lens), shuffled)
    V, H = cfg.vocab, cfg.hidden
    lm_bf16 = torch.from_numpy(np.ascontiguousarray(host["lm_head"]).view(np.int16)).cuda()
    lm_codes = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    lm_scales = torch.empty(V, dtype=torch.float32, device="cuda")
    M.mbg_quantize_fp8_rows(lm_bf16, V, H, lm_codes, lm_scales, torch.cuda.current_stream().cuda_stream)
    del lm_bf16
    experts = device_experts(cfg)
    dm = DeviceModel(cfg, host, pt, lm_fp8=(lm_codes, lm_scales), experts=experts, k_max=k_max)
    om = OracleModel(cfg, host, experts=lambda l, e, w: gen.expert_mxfp4(cfg, l, e, w),
                     lm_fp8=quantize_fp8_rows(host["lm_head"]), cache_experts=cache_experts)
    ocs = [OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim, "bf16") for _ in lens]
    for li in range(cfg.n_layers if cfg.prefill else 0):
        k, v = gen.kv_prefill_bf16(cfg, li)
        for b, (T, oc) in enumerate(zip(lens, ocs)):
            dm.prefill_bf16(li, k[:T], v[:T], seq=b)
            oc.k[li][:T] = k[:T]
            oc.v[li][:T] = v[:T]
    oc = ocs[0] if prefill_lens is None else ocs
    dm.init()
    return dm, om, oc


def build_draft(cfg, host, n_layers, target_dm=None):
    """(DeviceModel, OracleModel, OracleCache) of an early-exit draft: the
    target's first n_layers layers with its embedding, final norm and LM
    head (the same tensors), its cache prefilled like the target's first
    layers.  A routed target passes its DeviceModel for the experts and the
    FP8 LM head."""
    import torch
    from memory_bound_gemv_amd.device_model import DeviceModel
    dcfg = cfg.with_(n_layers=n_layers)
    import re
    keep = {k: v for k, v in host.items()
            if not re.match(r"l\d+\.", k) or int(k[1:].split(".")[0]) < n_layers}
    pt = gen.page_table(dcfg)
    if cfg.is_moe:
        dm = DeviceModel(dcfg, keep, pt, lm_fp8=(target_dm.lm_codes, target_dm.lm_scales),
                         experts=target_dm.experts[:n_layers])
        om = OracleModel(dcfg, keep, experts=lambda l, e, w: gen.expert_mxfp4(cfg, l, e, w),
                         lm_fp8=quantize_fp8_rows_cached(host))
    else:
        dm = DeviceModel(dcfg, keep, pt)
        om = OracleModel(dcfg, keep)
    oc = OracleCache(dcfg.n_layers, dcfg.max_pos, dcfg.n_kv_heads, dcfg.head_dim, "bf16")
    for li in range(n_layers if cfg.prefill else 0):
        k, v = gen.kv_prefill_bf16(cfg, li)
        dm.prefill_bf16(li, k, v)
        oc.k[li][:cfg.prefill] = k
        oc.v[li][:cfg.prefill] = v
    dm.init()
    return dm, om, oc


_FP8_LM = {}


def quantize_fp8_rows_cached(host):
    from oracle import quantize_fp8_rows
    key = id(host["lm_head"])
    if key not in _FP8_LM:
        _FP8_LM[key] = quantize_fp8_rows(host["lm_head"])
    return _FP8_LM[key]
