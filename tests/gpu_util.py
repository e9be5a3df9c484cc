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


def build_dense(cfg, shuffled=None, kv_dtype=None, kv_scales=None, k_max=None, host=None, block=1 << 16):
    """(DeviceModel, OracleModel, OracleCache) with identical weights and prefill.

    BF16 caches take their prefill as BF16 draws placed directly in both
    caches.  FP8 caches take float32 draws (made on the GPU) that each side
    rounds into its own cache: the library through mbg_kv_write, the oracle
    through its codec."""
    import torch
    from memory_bound_gemv_amd.device_model import DeviceModel
    kv_dtype = kv_dtype or cfg.kv_dtype
    host = host if host is not None else gen.dense_weights(cfg)
    pt = gen.page_table(cfg, shuffled)
    if kv_dtype == "fp8" and kv_scales is None:
        kv_scales = fp8_kv_scales(cfg, block)
    dm = DeviceModel(cfg, host, pt, kv_dtype=kv_dtype, kv_scales=kv_scales, k_max=k_max)
    om = OracleModel(cfg, host)
    oc = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim, kv_dtype)
    if kv_dtype == "fp8":
        oc.scales = np.asarray(kv_scales, dtype=np.float32).reshape(cfg.n_layers, cfg.n_kv_heads, 2)
    if cfg.prefill:
        for li in range(cfg.n_layers):
            k, v = gen.kv_prefill_bf16(cfg, li)
            if kv_dtype == "bf16":
                dm.prefill_bf16(li, k, v)
                oc.k[li][:cfg.prefill] = k
                oc.v[li][:cfg.prefill] = v
            else:
                for p0 in range(0, cfg.prefill, block):
                    n = min(block, cfg.prefill - p0)
                    k = gen.kv_prefill_f32_device(cfg, li, 0, p0, n, "cuda")
                    v = gen.kv_prefill_f32_device(cfg, li, 1, p0, n, "cuda")
                    dm.kv_write(li, p0, k, v)
                    oc.prefill_f32(li, p0, k.cpu().numpy(), v.cpu().numpy())
                torch.cuda.synchronize()
    dm.init()
    return dm, om, oc
