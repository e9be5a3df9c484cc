"""Workload shapes for the batch-1 decode path.

Five workloads, each a transformer (or one layer of it) at the sizes the
decode-speed pages discuss:

* ``tiny``   - 2-layer dense decoder, hidden 256; small enough that the CPU
  oracle finishes in well under a second per token.
* ``dense2b`` - 28-layer dense decoder of the 2B class (hidden 2048, 16/8
  heads of 128, SwiGLU 8192, vocab 32000) with a BF16 KV cache prefilled to
  4096 positions: the 2B FP16 model of the Kog article "Real-time LLM
  inference on standard GPUs: 3k tokens/s per request" (section on memory
  bandwidth as the bottleneck, worked bound for a 2B FP16 model).
* ``lmhead`` - the vocabulary projection alone, 157,184 x 2,560: the LM head
  of the 163.com article on batch-1 Ling-3.0-flash decode (section
  "optimisation 2: online FP8 LM head quantisation").
* ``moe``    - 42-layer mixture-of-experts stack with 512 routed experts
  (top-8) plus one shared expert, moe_intermediate 768, MXFP4 experts and an
  FP8 LM head: the shapes of the model in the same article (section "model
  and baseline configuration").
* ``longctx`` - the ``dense2b`` model with an FP8-e4m3 KV cache prefilled to
  200,000 positions in 64-token pages under a shuffled page table (the
  wmrh.cn report on Kimi-K3 long-context serving with vLLM and SGLang,
  sections on decode scaling and on the engines' configuration).

Only shapes and knobs live here; nothing in this module computes any part of
the decode step.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int            # dense SwiGLU width (0 for MoE layers)
    vocab: int
    n_experts: int = 0  # routed experts per layer (0 = dense)
    top_k: int = 0
    n_shared: int = 0
    moe_ffn: int = 0
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    kv_dtype: str = "bf16"        # "bf16" or "fp8"
    page_size: int = 64
    prefill: int = 0              # positions [0, prefill) hold synthetic K/V
    n_decode: int = 0             # decode steps the workload runs
    n_prompt: int = 0             # prompt tokens fed one per step (tiny only)
    lm_dtype: str = "bf16"        # "bf16" or "fp8"
    expert_dtype: str = "mxfp4"
    shuffled_pages: bool = False
    weight_sigma: float = 0.02
    k_max: int = 4                # widest verify window
    norm_gains: str = "ones"      # RMSNorm gains: "ones" (the configured 1.0) or
                                  # "random" (1 + 0.1 N(0, 1) per element, distinct per norm)
    layer_window: tuple = ()      # per-layer attention window W (0 = global); () = all global

    def window(self, layer: int) -> int:
        """Attention window of `layer`: position p attends [max(0, p - W + 1), p]; 0 = global."""
        return int(self.layer_window[layer]) if self.layer_window else 0

    @property
    def max_pos(self) -> int:
        """KV capacity in positions: prefill plus every decoded/prompt token."""
        return self.prefill + self.n_prompt + self.n_decode

    @property
    def n_pages(self) -> int:
        return -(-self.max_pos // self.page_size)

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


TINY = DecodeConfig(
    name="tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
    ffn=1024, vocab=4096, n_prompt=32, n_decode=16)

DENSE2B = DecodeConfig(
    name="dense2b", n_layers=28, hidden=2048, n_q_heads=16, n_kv_heads=8,
    head_dim=128, ffn=8192, vocab=32000, prefill=4096, n_decode=256)

# The LM head alone: only vocab/hidden matter.
LMHEAD = DecodeConfig(
    name="lmhead", n_layers=0, hidden=2560, n_q_heads=0, n_kv_heads=0,
    head_dim=0, ffn=0, vocab=157184)

MOE = DecodeConfig(
    name="moe", n_layers=42, hidden=2560, n_q_heads=32, n_kv_heads=4,
    head_dim=128, ffn=0, vocab=157184, n_experts=512, top_k=8, n_shared=1,
    moe_ffn=768, prefill=2048, n_decode=8, lm_dtype="fp8")

LONGCTX = DENSE2B.with_(name="longctx", kv_dtype="fp8", prefill=200000,
                        n_decode=64, shuffled_pages=True)

# The long-context workload with sliding-window layers: three of every four
# layers attend over the last 2,048 positions, the fourth globally (the
# Muse Spark Open article's model has 46 such layers of 62).
LONGCTX_SWA = LONGCTX.with_(name="longctx_swa",
                            layer_window=tuple(0 if li % 4 == 3 else 2048 for li in range(LONGCTX.n_layers)))

CONFIGS = {c.name: c for c in (TINY, DENSE2B, LMHEAD, MOE, LONGCTX, LONGCTX_SWA)}
