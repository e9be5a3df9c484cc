"""Batch-1 decode benchmark on one MI355X.

Workload: the 2B-class dense decoder (28 layers, hidden 2048, 16 query / 8 KV
heads of 128, SwiGLU 8192, vocab 32000, BF16 weights ~N(0, 0.02)), BF16 KV
cache prefilled with N(0, 1) to 4096 positions, greedy decode at batch 1.
One step = one decode_step call = one persistent-kernel launch that runs all
28 layers, the LM head and the argmax; the token of step i+1 is the argmax of
step i, read on the device (no host round trip inside the timed region).

Prints one JSON line (see the keys below).  --gpus N with N > 1 exits: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_kernel_dense2b_traffic.txt")

WORKLOADS = {
    "dense2b": "dense 2B decoder: 28 layers, hidden 2048, 16 query / 8 KV heads of 128, SwiGLU 8192, vocab 32000, "
               "BF16 weights N(0,0.02), BF16 KV prefilled N(0,1) to 4096 positions, batch 1, greedy decode at "
               "positions 4096..4351",
    "longctx": "dense 2B decoder (as dense2b) with an FP8-e4m3 KV cache (power-of-two per-head scales) prefilled "
               "N(0,1) to 200,000 positions in 64-token pages under a shuffled page table, batch 1, greedy decode "
               "at positions 200000..200063",
    "moe": "routed decoder: 42 layers, hidden 2560, 32 query / 4 KV heads of 128, 512 MXFP4 experts top-8 + 1 "
           "shared (moe_ffn 768), BF16 attention/router, FP8 LM head over vocab 157184, BF16 KV prefilled to 2048 "
           "positions, batch 1, greedy decode at positions 2048..2055",
}


def stored_traffic():
    """HBM bytes per launch of the decode-step kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain-copy calibration), or
    None when the summary is missing or was taken on other kernel sources."""
    from memory_bound_gemv_amd.build import source_digest
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_digest") != source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(cfg, pos: int) -> tuple[int, int]:
    """(weight bytes, KV bytes) one step at `pos` must read at least once.

    Weights: every BF16 attention matrix of every layer, the two norm gains
    per layer, the embedding row, the final norm and the LM head (BF16, or
    FP8 codes plus a float32 scale per row); dense layers add their three
    BF16 FFN matrices, routed layers the BF16 router plus the top-k and
    shared experts a token reads (MXFP4: half a byte per weight plus one
    E8M0 byte per 32).  KV: K and V of positions [0, pos] for every layer and
    KV head (the step's own K/V included), 2 bytes (BF16) or 1 (FP8)."""
    H, d = cfg.hidden, cfg.head_dim
    attn = 2 * (2 * H + (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d * H + H * cfg.n_q_heads * d)
    if cfg.is_moe:
        expert = 3 * cfg.moe_ffn * H * 17 // 32
        ffn = 2 * cfg.n_experts * H + (cfg.top_k + cfg.n_shared) * expert
    else:
        ffn = 2 * 3 * cfg.ffn * H
    lm = cfg.vocab * H + 4 * cfg.vocab if cfg.lm_dtype == "fp8" else 2 * cfg.vocab * H
    w = cfg.n_layers * (attn + ffn) + 2 * H + 2 * H + lm
    kv_el = 1 if cfg.kv_dtype == "fp8" else 2
    kv = (pos + 1) * cfg.n_layers * 2 * cfg.n_kv_heads * d * kv_el
    return w, kv


def fp8_pow2_scales(cfg, device, block=1 << 16):
    """Per (layer, KV head, K or V) power-of-two scale 2^ceil(log2(amax / 448))
    over the float32 prefill draws."""
    import numpy as np
    import torch

    from synth import gen
    sc = np.ones((cfg.n_layers, cfg.n_kv_heads, 2), dtype=np.float32)
    for li in range(cfg.n_layers):
        for kv in (0, 1):
            am = torch.zeros(cfg.n_kv_heads, dtype=torch.float32, device=device)
            for p0 in range(0, cfg.prefill, block):
                x = gen.kv_prefill_f32_device(cfg, li, kv, p0, min(block, cfg.prefill - p0), device)
                am = torch.maximum(am, x.abs().amax(dim=(0, 2)))
            sc[li, :, kv] = np.exp2(np.ceil(np.log2(am.double().cpu().numpy() / 448.0)))
    return sc


def build_device_model(cfg, host, dev):
    """The workload on the device: weights, prefilled KV cache, context."""
    import torch

    from memory_bound_gemv_amd import _mbg as M
    from memory_bound_gemv_amd.device_model import DeviceModel
    from synth import gen
    pt = gen.page_table(cfg)
    if cfg.is_moe:
        E, S, H, Mf, V = cfg.n_experts, cfg.n_shared, cfg.hidden, cfg.moe_ffn, cfg.vocab
        u8 = dict(dtype=torch.uint8, device=dev)
        experts = []
        for li in range(cfg.n_layers):
            d = dict(eg_codes=torch.empty((E, 2 * Mf, H // 2), **u8), eg_scales=torch.empty((E, 2 * Mf, H // 32), **u8),
                     ed_codes=torch.empty((E, H, Mf // 2), **u8), ed_scales=torch.empty((E, H, Mf // 32), **u8),
                     sg_codes=torch.empty((S, 2 * Mf, H // 2), **u8), sg_scales=torch.empty((S, 2 * Mf, H // 32), **u8),
                     sd_codes=torch.empty((S, H, Mf // 2), **u8), sd_scales=torch.empty((S, H, Mf // 32), **u8))
            gen.experts_mxfp4_torch(cfg, li, range(E), "gate_up", d["eg_codes"], d["eg_scales"])
            gen.experts_mxfp4_torch(cfg, li, range(E), "down", d["ed_codes"], d["ed_scales"])
            gen.experts_mxfp4_torch(cfg, li, range(E, E + S), "gate_up", d["sg_codes"], d["sg_scales"])
            gen.experts_mxfp4_torch(cfg, li, range(E, E + S), "down", d["sd_codes"], d["sd_scales"])
            experts.append(d)
        import numpy as np
        lm_bf16 = torch.from_numpy(np.ascontiguousarray(host["lm_head"]).view(np.int16)).to(dev)
        lm_codes = torch.empty((V, H), **u8)
        lm_scales = torch.empty(V, dtype=torch.float32, device=dev)
        M.mbg_quantize_fp8_rows(lm_bf16, V, H, lm_codes, lm_scales, torch.cuda.current_stream(dev).cuda_stream)
        dm = DeviceModel(cfg, host, pt, lm_fp8=(lm_codes, lm_scales), experts=experts, device=dev, k_max=1)
    elif cfg.kv_dtype == "fp8":
        dm = DeviceModel(cfg, host, pt, kv_dtype="fp8", kv_scales=fp8_pow2_scales(cfg, dev), device=dev, k_max=1)
    else:
        dm = DeviceModel(cfg, host, pt, device=dev, k_max=1)
    for li in range(cfg.n_layers):
        if cfg.kv_dtype == "fp8":
            blk = 1 << 16
            for p0 in range(0, cfg.prefill, blk):
                n = min(blk, cfg.prefill - p0)
                dm.kv_write(li, p0, gen.kv_prefill_f32_device(cfg, li, 0, p0, n, dev),
                            gen.kv_prefill_f32_device(cfg, li, 1, p0, n, dev))
        else:
            k, v = gen.kv_prefill_bf16(cfg, li)
            dm.prefill_bf16(li, k, v)
    dm.init()
    return dm


def cpu_baseline(cfg, host, steps: int = 3):
    """Time the CPU oracle (float64, as it stands) on a few decode steps."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import OracleCache, OracleModel
    from synth import gen

    om = OracleModel(cfg, host)
    oc = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    for li in range(cfg.n_layers):
        k, v = gen.kv_prefill_bf16(cfg, li)
        oc.k[li][:cfg.prefill] = k
        oc.v[li][:cfg.prefill] = v
    toks = gen.prompt_tokens(cfg, steps + 1)
    t0 = time.perf_counter()
    om.step(oc, int(toks[0]), cfg.prefill)          # dequantises and caches the weights
    t_first = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(steps):
        om.step(oc, int(toks[i + 1]), cfg.prefill + 1 + i)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": steps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{steps} float64 oracle decode steps of the same workload at positions "
                       f"{cfg.prefill + 1}..{cfg.prefill + steps} after one untimed step "
                       f"({t_first:.1f} s) that converted and cached the weights; "
                       f"host cpu_count {os.cpu_count()}")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace", default="",
                    help="after the timed region, run one traced step and save its per-task stamps (.npy)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    ap.add_argument("--workload", default="dense2b", choices=["dense2b", "longctx", "moe"],
                    help="dense2b (default, the headline line), longctx (FP8 KV at 200K positions) "
                         "or moe (42-layer routed model); only dense2b carries the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path has no "
              "multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from synth import CONFIGS, gen

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    host = gen.dense_weights(cfg)
    dm = build_device_model(cfg, host, dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    info = dm.info()

    stream = torch.cuda.current_stream(dev)
    buf = torch.tensor([int(gen.prompt_tokens(cfg, 1)[0])], dtype=torch.int32, device=dev)
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device=dev)
    n_slots = cfg.n_decode                     # positions prefill .. prefill + n_decode - 1, cycled
    pos_of = lambda i: cfg.prefill + (i % n_slots)

    for i in range(args.warmup):
        dm.step(buf, pos_of(i), logits, buf)
    torch.cuda.synchronize()
    if dm.status() != 0:
        raise RuntimeError("device status after warm-up")

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        dm.step(buf, pos_of(args.warmup + i), logits, buf)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st = dm.status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    tok_s = args.steps / (ms / 1e3)

    wbytes, _ = algorithmic_bytes(cfg, 0)
    kv_avg = float(np.mean([algorithmic_bytes(cfg, pos_of(args.warmup + i))[1] for i in range(args.steps)]))
    step_bytes = wbytes + kv_avg
    achieved = step_bytes / (ms_per_step / 1e3) / 1e9

    if args.trace:
        from memory_bound_gemv_amd import _mbg as M
        M.mbg_set_trace(dm.ctx, True)
        dm.step(buf, pos_of(args.warmup + args.steps), logits, buf)
        rec = M.mbg_read_trace(dm.ctx, info.n_tasks)
        M.mbg_set_trace(dm.ctx, False)
        np.save(args.trace, rec)
        np.save(args.trace.replace(".npy", "_meta.npy"),
                np.array([info.clock_khz, info.grid, cfg.n_layers], dtype=np.int64))

    if args.copy_probe_mib:
        n = args.copy_probe_mib * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": "batch-1 decode tokens/s and achieved HBM GB/s (MBU % of peak) on 1 MI355X",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.workload],
            "weight_dtype": "bf16+mxfp4 experts+fp8 lm head" if cfg.is_moe else "bf16",
            "kv_dtype": cfg.kv_dtype, "accumulate": "fp32",
            "global_batch": 1, "seq_len": cfg.prefill, "parallelism": "none (1 GPU)",
            "kernel": info.variant.decode(), "grid": info.grid, "launches_per_step": info.launches_per_step,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": stored_traffic() if args.workload == "dense2b" else None,
        },
        "bytes_per_step": {"weights": wbytes, "kv_avg": round(kv_avg), "total": round(step_bytes)},
        "bound_tokens_s": round(PEAK_HBM_GBS * 1e9 / step_bytes, 1),
        "wall_tokens_s": round(args.steps / wall, 2),
        "setup_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline and args.workload == "dense2b":
        out["cpu_baseline"] = cpu_baseline(cfg, host)
    print(json.dumps(out), flush=True)
    dm.close()


if __name__ == "__main__":
    main()
