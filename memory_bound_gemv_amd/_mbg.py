"""ctypes binding of libmbg.so: the C-ABI declared in include/mbg.h, with the
same function names.  Argument marshalling only; every step of the decode path
runs in the HIP library.  Importing this module fails loudly when the library
has not been built."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmbg.so")

MBG_OK = 0
MBG_E_INVALID_ARG = -1
MBG_E_UNSUPPORTED = -2
MBG_E_DTYPE_MISMATCH = -3
MBG_E_RANGE = -4
MBG_E_WORKSPACE = -5
MBG_E_HIP = -6
MBG_E_TIMEOUT = -7

MBG_BF16 = 1
MBG_FP8_E4M3 = 2
MBG_MXFP4 = 3
MBG_FP32 = 4

DTYPES = {"bf16": MBG_BF16, "fp8": MBG_FP8_E4M3, "mxfp4": MBG_MXFP4, "fp32": MBG_FP32}


class MbgError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mbg error {code}: {msg}")
        self.code = code


class mbg_tensor(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("n", C.c_int32), ("rows", C.c_int64), ("cols", C.c_int64),
                ("data", C.c_void_p), ("scale", C.c_void_p)]


_LAYER_FIELDS = ["attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down",
                 "w_router", "exp_gate_up", "exp_down", "sh_gate_up", "sh_down"]


class mbg_layer(C.Structure):
    _fields_ = [(f, mbg_tensor) for f in _LAYER_FIELDS]


class mbg_weights(C.Structure):
    _fields_ = [("layers", C.POINTER(mbg_layer)), ("embed", mbg_tensor), ("final_norm", mbg_tensor),
                ("lm_head", mbg_tensor)]


class mbg_kv(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("n_pages", C.c_int32), ("pool", C.c_void_p),
                ("page_table", C.c_void_p), ("scales", C.c_void_p), ("n_seqs", C.c_int32)]


class mbg_config(C.Structure):
    _fields_ = [(f, C.c_int32) for f in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                          "vocab", "n_experts", "top_k", "n_shared", "moe_ffn")] + [
        ("rope_theta", C.c_float), ("rms_eps", C.c_float), ("page_size", C.c_int32), ("max_pos", C.c_int32),
        ("k_max", C.c_int32), ("layer_window", C.POINTER(C.c_int32))]


class mbg_info(C.Structure):
    _fields_ = [(f, C.c_int32) for f in ("grid", "block", "n_tasks", "launches_per_step", "lm_dtype", "kv_dtype",
                                          "expert_dtype", "attn_dtype", "attn_splits", "attn_local", "trace",
                                          "verify_path")] + [
        ("weight_bytes_per_step", C.c_int64), ("workspace_bytes", C.c_int64), ("clock_khz", C.c_int64),
        ("variant", C.c_char * 64)]


class mbg_ctx(C.Structure):
    pass


CTX_P = C.POINTER(mbg_ctx)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with memory_bound_gemv_amd.build.build() "
                          "(the decode path has no fallback)")
    # The library and the caller's PyTorch must share one HIP runtime: PyTorch
    # ships its own, and when that is loaded first the library's dependency
    # resolves to it.  Loaded the other way round the process holds two
    # runtimes, and the library's sees no device once PyTorch has claimed it
    # (measured: hipGetDevice fails in mbg_decode_init).  So PyTorch, when
    # installed, is imported before the library is loaded.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = C.CDLL(LIB_PATH)
    sig = {
        "mbg_workspace_size": (C.c_int, [C.POINTER(mbg_config), C.POINTER(C.c_size_t)]),
        "mbg_validate": (C.c_int, [C.POINTER(mbg_config), C.POINTER(mbg_weights), C.POINTER(mbg_kv)]),
        "mbg_counter_bytes": (C.c_int, [C.POINTER(mbg_config), C.POINTER(C.c_size_t)]),
        "mbg_decode_init": (C.c_int, [C.POINTER(mbg_config), C.POINTER(mbg_weights), C.POINTER(mbg_kv),
                                      C.c_void_p, C.c_size_t, C.c_void_p, C.c_size_t, C.c_void_p,
                                      C.POINTER(CTX_P)]),
        "mbg_decode_step": (C.c_int, [CTX_P, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
        "mbg_decode_verify": (C.c_int, [CTX_P, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
        "mbg_decode_steps": (C.c_int, [CTX_P, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
        "mbg_decode_batch": (C.c_int, [CTX_P, C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                       C.c_void_p, C.c_void_p]),
        "mbg_spec_round": (C.c_int, [CTX_P, CTX_P, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                                     C.c_void_p]),
        "mbg_get_status": (C.c_int, [CTX_P]),
        "mbg_query": (C.c_int, [CTX_P, C.POINTER(mbg_info)]),
        "mbg_set_timeout_us": (C.c_int, [CTX_P, C.c_int64]),
        "mbg_set_trace": (C.c_int, [CTX_P, C.c_int]),
        "mbg_set_verify_path": (C.c_int, [CTX_P, C.c_int]),
        "mbg_read_trace": (C.c_int, [CTX_P, C.c_void_p, C.c_size_t, C.POINTER(C.c_size_t)]),
        "mbg_read_routing": (C.c_int, [CTX_P, C.c_int32, C.c_void_p, C.c_void_p, C.POINTER(C.c_int32)]),
        "mbg_last_error": (C.c_char_p, []),
        "mbg_destroy": (None, [CTX_P]),
        "mbg_lm_head_workspace_size": (C.c_int, [C.c_int32, C.POINTER(C.c_size_t)]),
        "mbg_lm_head": (C.c_int, [C.POINTER(mbg_tensor), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_size_t, C.c_void_p]),
        "mbg_lm_head_noalloc": (C.c_int, [C.POINTER(mbg_tensor), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                          C.c_void_p]),
        "mbg_quantize_fp8_rows": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_void_p,
                                            C.c_void_p]),
        "mbg_kv_write": (C.c_int, [C.POINTER(mbg_config), C.POINTER(mbg_kv), C.c_int32, C.c_int32, C.c_int32,
                                   C.c_void_p, C.c_void_p, C.c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("mbg_workspace_size", "mbg_counter_bytes", "mbg_validate", "mbg_decode_init", "mbg_decode_step",
            "mbg_decode_verify", "mbg_decode_steps", "mbg_decode_batch", "mbg_spec_round",
            "mbg_get_status", "mbg_query", "mbg_set_timeout_us", "mbg_set_verify_path", "mbg_set_trace",
            "mbg_read_trace",
            "mbg_read_routing", "mbg_last_error", "mbg_destroy",
            "mbg_lm_head_workspace_size", "mbg_lm_head", "mbg_lm_head_noalloc", "mbg_quantize_fp8_rows",
            "mbg_kv_write")


def _check(rc: int) -> int:
    if rc != MBG_OK:
        raise MbgError(rc, mbg_last_error())
    return rc


def _ptr(x):
    """Device/host address of a torch tensor, an int, or None (NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


# --------------------------------------------------------------------------- marshalling helpers

def make_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_experts=0, top_k=0,
                n_shared=0, moe_ffn=0, rope_theta=1e4, rms_eps=1e-6, page_size=64, max_pos=1, k_max=1,
                layer_window=None):
    """layer_window: per-layer attention windows (0 = global) or None.  The
    returned struct keeps the array alive (``_keep``)."""
    cfg = mbg_config(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_experts, top_k, n_shared,
                     moe_ffn, rope_theta, rms_eps, page_size, max_pos, k_max, None)
    if layer_window is not None:
        arr = (C.c_int32 * n_layers)(*[int(w) for w in layer_window])
        cfg.layer_window = C.cast(arr, C.POINTER(C.c_int32))
        cfg._keep = arr
    return cfg


def make_tensor(data, dtype, rows, cols, n=1, scale=None) -> mbg_tensor:
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    return mbg_tensor(dtype, n, rows, cols, _ptr(data), _ptr(scale))


class WeightSet:
    """Holds an mbg_weights struct and the ctypes objects it points into."""

    def __init__(self, layers, embed, final_norm, lm_head):
        self._layers = (mbg_layer * max(1, len(layers)))(*layers)
        self.struct = mbg_weights(self._layers, embed, final_norm, lm_head)


def make_layer(**tensors) -> mbg_layer:
    lay = mbg_layer()
    for k, v in tensors.items():
        if k not in _LAYER_FIELDS:
            raise KeyError(k)
        setattr(lay, k, v)
    return lay


def make_kv(dtype, n_pages, pool, page_table, scales=None, n_seqs=1) -> mbg_kv:
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    return mbg_kv(dtype, n_pages, _ptr(pool), _ptr(page_table), _ptr(scales), n_seqs)


# --------------------------------------------------------------------------- the C-ABI, same names

def mbg_last_error() -> str:
    return _lib.mbg_last_error().decode()


def mbg_workspace_size(cfg: mbg_config) -> int:
    n = C.c_size_t(0)
    _check(_lib.mbg_workspace_size(C.byref(cfg), C.byref(n)))
    return n.value


def mbg_counter_bytes(cfg: mbg_config) -> int:
    n = C.c_size_t(0)
    _check(_lib.mbg_counter_bytes(C.byref(cfg), C.byref(n)))
    return n.value


def mbg_validate(cfg: mbg_config, weights=None, kv=None) -> int:
    """Returns the library's code (0 or negative); does not raise."""
    w = C.byref(weights.struct) if weights is not None else None
    k = C.byref(kv) if kv is not None else None
    return _lib.mbg_validate(C.byref(cfg), w, k)


def mbg_decode_init(cfg, weights: WeightSet, kv, workspace, ws_bytes: int, counters, counter_bytes: int,
                    stream: int):
    ctx = CTX_P()
    _check(_lib.mbg_decode_init(C.byref(cfg), C.byref(weights.struct), C.byref(kv), _ptr(workspace), ws_bytes,
                                _ptr(counters), counter_bytes, stream, C.byref(ctx)))
    return ctx


def mbg_decode_step(ctx, token, pos: int, logits, argmax) -> None:
    _check(_lib.mbg_decode_step(ctx, _ptr(token), pos, _ptr(logits), _ptr(argmax)))


def mbg_decode_verify(ctx, tokens, k: int, pos: int, logits, argmax) -> None:
    _check(_lib.mbg_decode_verify(ctx, _ptr(tokens), k, pos, _ptr(logits), _ptr(argmax)))


def mbg_decode_steps(ctx, token, n_steps: int, pos: int, logits, argmax) -> None:
    _check(_lib.mbg_decode_steps(ctx, _ptr(token), n_steps, pos, _ptr(logits), _ptr(argmax)))


def mbg_decode_batch(ctx, tokens, n: int, seq, pos, logits, argmax) -> None:
    """seq, pos: host sequences of n ints (page-table rows, positions)."""
    sq = (C.c_int32 * n)(*[int(v) for v in seq])
    ps = (C.c_int32 * n)(*[int(v) for v in pos])
    _check(_lib.mbg_decode_batch(ctx, _ptr(tokens), n, sq, ps, _ptr(logits), _ptr(argmax)))


# mbg_spec_state: int32 words pos, n_emitted, n_accepted, n_rounds, window[8]
SPEC_STATE_WORDS = 12


def mbg_spec_round(target, draft, k: int, state, next_state, emit, emit_cap: int, logits=None) -> None:
    _check(_lib.mbg_spec_round(target, draft, k, _ptr(state), _ptr(next_state), _ptr(emit), emit_cap,
                               _ptr(logits)))


def mbg_get_status(ctx) -> int:
    return _lib.mbg_get_status(ctx)


def mbg_query(ctx) -> mbg_info:
    info = mbg_info()
    _check(_lib.mbg_query(ctx, C.byref(info)))
    return info


def mbg_set_timeout_us(ctx, us: int) -> None:
    _check(_lib.mbg_set_timeout_us(ctx, us))


MBG_PATH_FMA = 0
MBG_PATH_MFMA = 1


def mbg_set_verify_path(ctx, path: int) -> None:
    _check(_lib.mbg_set_verify_path(ctx, path))


def mbg_set_trace(ctx, on: bool) -> None:
    _check(_lib.mbg_set_trace(ctx, 1 if on else 0))


def mbg_read_trace(ctx, n_tasks: int):
    """Trace records of the last step as a uint64 numpy array [n][8]."""
    import numpy as np
    buf = np.zeros((n_tasks, 8), dtype=np.uint64)
    n = C.c_size_t(0)
    _check(_lib.mbg_read_trace(ctx, buf.ctypes.data, n_tasks, C.byref(n)))
    return buf[: n.value]


def mbg_read_routing(ctx, layer: int, k_max: int, top_k: int):
    """(expert ids int32 [ncol][top_k], weights float32 [ncol][top_k]) of the
    last call's routing in `layer`."""
    import numpy as np
    idx = np.zeros(k_max * top_k, dtype=np.int32)
    w = np.zeros(k_max * top_k, dtype=np.float32)
    n = C.c_int32(0)
    _check(_lib.mbg_read_routing(ctx, layer, idx.ctypes.data, w.ctypes.data, C.byref(n)))
    return idx[: n.value * top_k].reshape(n.value, top_k), w[: n.value * top_k].reshape(n.value, top_k)


def mbg_destroy(ctx) -> None:
    _lib.mbg_destroy(ctx)


def mbg_lm_head_workspace_size(k: int) -> int:
    n = C.c_size_t(0)
    _check(_lib.mbg_lm_head_workspace_size(k, C.byref(n)))
    return n.value


def mbg_lm_head(w: mbg_tensor, x, k: int, logits, argmax, workspace, ws_bytes: int, stream: int) -> None:
    _check(_lib.mbg_lm_head(C.byref(w), _ptr(x), k, _ptr(logits), _ptr(argmax), _ptr(workspace), ws_bytes,
                            stream))


def mbg_lm_head_noalloc(w: mbg_tensor, x, k: int, logits, argmax, stream: int) -> None:
    _check(_lib.mbg_lm_head_noalloc(C.byref(w), _ptr(x), k, _ptr(logits), _ptr(argmax), stream))


def mbg_quantize_fp8_rows(w, rows: int, cols: int, codes, scales, stream: int) -> None:
    _check(_lib.mbg_quantize_fp8_rows(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), stream))


def mbg_kv_write(cfg, kv, layer: int, pos0: int, n: int, k, v, stream: int) -> None:
    _check(_lib.mbg_kv_write(C.byref(cfg), C.byref(kv), layer, pos0, n, _ptr(k), _ptr(v), stream))
