"""Device-side plumbing around the C-ABI: upload host arrays into torch
device tensors, describe them to the library, own the KV pool and the
workspace, and forward step/verify calls.  No decode arithmetic happens here
(PyTorch provides device memory and the stream; the HIP library does the
work)."""
from __future__ import annotations

import ctypes
import threading

import numpy as np
import torch

from . import _mbg as M

_HIP_DEVICE_MALLOC_UNCACHED = 0x3   # hipDeviceMallocUncached (hip_runtime_api.h)


def _hip_runtime() -> ctypes.CDLL:
    """The HIP runtime this process already uses (the one torch loaded and
    libmbg.so links against), opened by its path so that no second runtime
    is loaded."""
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in path and path.startswith("/"):
                return ctypes.CDLL(path)
    raise RuntimeError("the HIP runtime is not loaded (import torch and use a GPU first)")


class UncachedPool:
    """Dependency-counter blocks in device memory that the L2 does not cache.

    The decode kernel polls its counters with cache-bypassing scalar loads,
    which see other XCDs' updates only in uncached memory; torch cannot
    allocate such memory, so it comes from the HIP runtime directly.  A block
    that a kernel has read is not freed before the process ends: released
    blocks go back to this pool and later contexts on the same device reuse
    them."""

    def __init__(self):
        self._free = {}          # device index -> [(bytes, address)]
        self._lock = threading.Lock()
        self._hip = None

    def acquire(self, nbytes: int, device: torch.device) -> tuple[int, int]:
        dev = device.index if device.index is not None else torch.cuda.current_device()
        with self._lock:
            free = self._free.setdefault(dev, [])
            for i, (n, addr) in enumerate(free):
                if n >= nbytes:
                    del free[i]
                    return addr, n
            if self._hip is None:
                self._hip = _hip_runtime()
                self._hip.hipExtMallocWithFlags.restype = ctypes.c_int
                self._hip.hipExtMallocWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t,
                                                            ctypes.c_uint]
            nbytes = (nbytes + 4095) // 4096 * 4096
            p = ctypes.c_void_p()
            with torch.cuda.device(dev):
                rc = self._hip.hipExtMallocWithFlags(ctypes.byref(p), nbytes, _HIP_DEVICE_MALLOC_UNCACHED)
            if rc != 0 or not p.value:
                raise RuntimeError(f"hipExtMallocWithFlags(uncached, {nbytes}) failed with {rc}")
            return p.value, nbytes

    def release(self, addr: int, nbytes: int, device: torch.device) -> None:
        dev = device.index if device.index is not None else torch.cuda.current_device()
        with self._lock:
            self._free.setdefault(dev, []).append((nbytes, addr))


UNCACHED = UncachedPool()


def _dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to(device)


class DeviceModel:
    """One decoder on one GPU.

    cfg: any object with the shape attributes of ``synth.configs.DecodeConfig``.
    host: dict of host arrays named like ``embed``, ``final_norm``, ``lm_head``,
    ``l{i}.{attn_norm,wq,wk,wv,wo,ffn_norm,w_gate,w_up,w_down}`` (BF16 bits as
    uint16).  lm_fp8: optional (codes uint8 [V][H], scales f32 [V]) given as
    device tensors, replacing the BF16 LM head.
    page_table: host int32 [n_pages] logical -> physical page.
    experts: MoE only, per layer a dict of device uint8 tensors: eg_codes
    [E][2M][H/2], eg_scales [E][2M][H/32], ed_codes [E][H][M/2], ed_scales
    [E][H][M/32] and the same for the shared experts (sg_*, sd_*, n = S).
    """

    def __init__(self, cfg, host: dict, page_table: np.ndarray, kv_dtype: str = "bf16", kv_scales=None,
                 lm_fp8=None, device="cuda", k_max: int | None = None, experts=None):
        self.cfg = cfg
        self.device = torch.device(device)
        self.k_max = k_max or cfg.k_max
        self.t = {k: _dev(v, self.device) for k, v in host.items()}
        # The library keeps raw pointers into every tensor it is given: hold
        # references for as long as the context lives.
        self.experts = experts
        H, d = cfg.hidden, cfg.head_dim
        bf = "bf16"

        def T(name, rows, cols):
            return M.make_tensor(self.t[name], bf, rows, cols)

        layers = []
        for i in range(cfg.n_layers):
            p = f"l{i}."
            lay = dict(
                attn_norm=T(p + "attn_norm", 1, H), ffn_norm=T(p + "ffn_norm", 1, H),
                wq=T(p + "wq", cfg.n_q_heads * d, H), wk=T(p + "wk", cfg.n_kv_heads * d, H),
                wv=T(p + "wv", cfg.n_kv_heads * d, H), wo=T(p + "wo", H, cfg.n_q_heads * d))
            if not cfg.is_moe:
                lay.update(w_gate=T(p + "w_gate", cfg.ffn, H), w_up=T(p + "w_up", cfg.ffn, H),
                           w_down=T(p + "w_down", H, cfg.ffn))
            else:
                e = experts[i]
                E, S, Mf = cfg.n_experts, cfg.n_shared, cfg.moe_ffn
                lay.update(
                    w_router=T(p + "w_router", E, H),
                    exp_gate_up=M.make_tensor(e["eg_codes"], "mxfp4", 2 * Mf, H, n=E, scale=e["eg_scales"]),
                    exp_down=M.make_tensor(e["ed_codes"], "mxfp4", H, Mf, n=E, scale=e["ed_scales"]))
                if S:
                    lay.update(
                        sh_gate_up=M.make_tensor(e["sg_codes"], "mxfp4", 2 * Mf, H, n=S, scale=e["sg_scales"]),
                        sh_down=M.make_tensor(e["sd_codes"], "mxfp4", H, Mf, n=S, scale=e["sd_scales"]))
            layers.append(M.make_layer(**lay))
        if lm_fp8 is not None:
            self.lm_codes, self.lm_scales = lm_fp8
            lm = M.make_tensor(self.lm_codes, "fp8", cfg.vocab, H, scale=self.lm_scales)
        else:
            lm = T("lm_head", cfg.vocab, H)
        self.weights = M.WeightSet(layers, T("embed", cfg.vocab, H), T("final_norm", 1, H), lm)

        # KV pool [L][P][2][Hkv][page][d]
        self.n_pages = int(page_table.max()) + 1 if page_table.size else 1
        self.n_pages = max(self.n_pages, cfg.n_pages)
        el = torch.int16 if kv_dtype == "bf16" else torch.uint8
        self.pool = torch.zeros((cfg.n_layers, self.n_pages, 2, cfg.n_kv_heads, cfg.page_size, d), dtype=el,
                                device=self.device)
        # one row per sequence (a 1-D table is the one sequence 0)
        self.page_table_host = np.asarray(page_table, dtype=np.int32)
        self.n_seqs = self.page_table_host.shape[0] if self.page_table_host.ndim == 2 else 1
        self.page_table = torch.from_numpy(self.page_table_host).to(self.device)
        self.kv_scales = None
        if kv_dtype == "fp8":
            self.kv_scales = torch.as_tensor(np.asarray(kv_scales, dtype=np.float32)).to(self.device).contiguous()
        self.kv = M.make_kv(kv_dtype, self.n_pages, self.pool, self.page_table, self.kv_scales, self.n_seqs)
        self.kv_dtype = kv_dtype

        self.mcfg = M.make_config(cfg.n_layers, H, cfg.n_q_heads, cfg.n_kv_heads, d, cfg.ffn, cfg.vocab,
                                  cfg.n_experts, cfg.top_k, cfg.n_shared, cfg.moe_ffn, cfg.rope_theta,
                                  cfg.rms_eps, cfg.page_size, cfg.max_pos, self.k_max,
                                  layer_window=list(cfg.layer_window) if cfg.layer_window else None)
        self.ws_bytes = M.mbg_workspace_size(self.mcfg)
        self.ws = torch.zeros(self.ws_bytes // 4 + 64, dtype=torch.int32, device=self.device)
        self.ctr_bytes = M.mbg_counter_bytes(self.mcfg)
        self.ctr = None           # (address, bytes) of the uncached counter block while a context lives
        self.stream = torch.cuda.current_stream(self.device)
        self.ctx = None

    # ------------------------------------------------------------------ KV prefill
    def _row(self, seq: int) -> torch.Tensor:
        return self.page_table[seq] if self.page_table.dim() == 2 else self.page_table

    def prefill_bf16(self, layer: int, k_bits: np.ndarray, v_bits: np.ndarray, seq: int = 0) -> None:
        """Place logical BF16 K/V [T][Hkv][d] of positions [0, T) of sequence
        `seq` into its pages."""
        cfg = self.cfg
        T = k_bits.shape[0]
        P = cfg.page_size
        npg = -(-T // P)
        for which, src in ((0, k_bits), (1, v_bits)):
            full = np.zeros((npg * P, cfg.n_kv_heads, cfg.head_dim), dtype=np.uint16)
            full[:T] = src
            blk = torch.from_numpy(full.view(np.int16)).to(self.device)
            blk = blk.view(npg, P, cfg.n_kv_heads, cfg.head_dim).permute(0, 2, 1, 3)
            phys = self._row(seq)[:npg].long()
            if T % P:  # keep slots of the last page beyond T untouched
                last = phys[-1]
                keep = self.pool[layer, last, which, :, T % P:, :].clone()
            self.pool[layer, phys, which] = blk
            if T % P:
                self.pool[layer, last, which, :, T % P:, :] = keep

    def kv_write(self, layer: int, pos0: int, k: torch.Tensor, v: torch.Tensor, seq: int = 0) -> None:
        """Quantising write through the library (cache dtype rounding) into
        sequence `seq`'s pages."""
        kv = self.kv if seq == 0 else M.make_kv(self.kv_dtype, self.n_pages, self.pool, self._row(seq),
                                                self.kv_scales)
        M.mbg_kv_write(self.mcfg, kv, layer, pos0, k.shape[0], k, v, self.stream.cuda_stream)

    # ------------------------------------------------------------------ decode
    def init(self) -> None:
        self.ctr = UNCACHED.acquire(self.ctr_bytes, self.device)
        try:
            self.ctx = M.mbg_decode_init(self.mcfg, self.weights, self.kv, self.ws, self.ws_bytes, self.ctr[0],
                                         self.ctr[1], self.stream.cuda_stream)
        except Exception:
            UNCACHED.release(*self.ctr, self.device)
            self.ctr = None
            raise

    def info(self):
        return M.mbg_query(self.ctx)

    def step(self, token: torch.Tensor, pos: int, logits: torch.Tensor | None, argmax: torch.Tensor) -> None:
        M.mbg_decode_step(self.ctx, token, pos, logits, argmax)

    def steps(self, token: torch.Tensor, n_steps: int, pos: int, logits, argmax: torch.Tensor) -> None:
        """n_steps greedy steps in one launch (argmax [n_steps], logits [n_steps][V] or None)."""
        M.mbg_decode_steps(self.ctx, token, n_steps, pos, logits, argmax)

    def verify(self, tokens: torch.Tensor, pos: int, logits, argmax) -> None:
        M.mbg_decode_verify(self.ctx, tokens, tokens.numel(), pos, logits, argmax)

    def batch(self, tokens: torch.Tensor, seq, pos, logits, argmax) -> None:
        """One step of len(seq) independent sequences: column i is token
        tokens[i] of sequence seq[i] at position pos[i]."""
        M.mbg_decode_batch(self.ctx, tokens, len(seq), seq, pos, logits, argmax)

    def spec_round(self, draft: "DeviceModel", k: int, state: torch.Tensor, next_state: torch.Tensor,
                   emit: torch.Tensor, logits=None) -> None:
        """One speculative round: `draft` proposes k tokens, this model
        verifies the window and accepts on the device (state, next_state:
        int32 [12] device tensors; emit: int32 device tensor)."""
        M.mbg_spec_round(self.ctx, draft.ctx, k, state, next_state, emit, emit.numel(), logits)

    def status(self) -> int:
        return M.mbg_get_status(self.ctx)

    def routing(self, layer: int):
        """(expert ids [ncol][top_k], weights [ncol][top_k]) of the last call."""
        return M.mbg_read_routing(self.ctx, layer, self.k_max, self.cfg.top_k)

    def close(self) -> None:
        if self.ctx is not None:
            M.mbg_destroy(self.ctx)     # waits for the context's stream
            self.ctx = None
        if self.ctr is not None:
            UNCACHED.release(*self.ctr, self.device)
            self.ctr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ inspection
    def cache_logical(self, layer: int, upto: int):
        """K, V of positions [0, upto) gathered back from the pages (host arrays)."""
        cfg = self.cfg
        P = cfg.page_size
        npg = -(-upto // P)
        phys = self.page_table[:npg].long()
        out = []
        for which in (0, 1):
            blk = self.pool[layer, phys, which]                  # [npg][Hkv][P][d]
            blk = blk.permute(0, 2, 1, 3).reshape(npg * P, cfg.n_kv_heads, cfg.head_dim)[:upto]
            a = blk.cpu().numpy()
            out.append(a.view(np.uint16) if a.dtype == np.int16 else a)
        return out[0], out[1]
