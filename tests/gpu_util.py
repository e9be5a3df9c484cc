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


def build_dense(cfg, shuffled=None, kv_dtype="bf16", kv_scales=None, k_max=None, host=None):
    """(DeviceModel, OracleModel, OracleCache) with identical weights and prefill."""
    import torch  # noqa: F401
    from memory_bound_gemv_amd.device_model import DeviceModel
    host = host if host is not None else gen.dense_weights(cfg)
    pt = gen.page_table(cfg, shuffled)
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
                raise NotImplementedError
    dm.init()
    return dm, om, oc
