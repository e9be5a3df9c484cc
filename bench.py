"""Batch-1 decode benchmark on one MI355X.

Default workload: the routed decoder (42 layers, hidden 2560, 32 query / 4 KV
heads of 128, 512 MXFP4 experts top-8 plus one shared expert, moe_ffn 768,
BF16 attention and router, FP8 LM head over a 157,184-token vocabulary), KV
prefilled to 2048 positions, greedy decode at batch 1 -- the largest
configuration of the workload set that fits one GPU.  One step = one
decode_step call = one persistent-kernel launch that runs every layer, the LM
head and the argmax; the token of step i+1 is the argmax of step i, read on
the device (no host round trip inside the timed region).  The same run times
the 4-token verify window.

Other workloads (--workload): dense2b, longctx (FP8 KV at 200,000
positions), lmhead (the LM head GEMV alone, --lm-dtype bf16|fp8, --k 1..4).

Prints one JSON line.  --gpus N with N > 1 exits: the decode path runs on one
GPU.
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
METRIC = "batch-1 decode tokens/s and achieved HBM GB/s (MBU % of peak) on 1 MI355X"

WORKLOADS = {
    "dense2b": "dense 2B decoder: 28 layers, hidden 2048, 16 query / 8 KV heads of 128, SwiGLU 8192, vocab 32000, "
               "BF16 weights N(0,0.02), BF16 KV prefilled N(0,1) to 4096 positions, batch 1, greedy decode at "
               "positions 4096..4351",
    "longctx": "dense 2B decoder (as dense2b) with an FP8-e4m3 KV cache (power-of-two per-head scales) prefilled "
               "N(0,1) to 200,000 positions in 64-token pages under a shuffled page table, batch 1, greedy decode "
               "at positions 200000..200063",
    "longctx_swa": "long-context workload (as longctx: FP8 KV at 200,000 positions, shuffled pages) with "
                   "sliding-window layers: layers 4i..4i+2 attend over the last 2,048 positions, layer 4i+3 "
                   "globally, batch 1, greedy decode at positions 200000..200063",
    "moe": "routed decoder: 42 layers, hidden 2560, 32 query / 4 KV heads of 128, 512 MXFP4 experts top-8 + 1 "
           "shared (moe_ffn 768), BF16 attention/router, FP8 LM head over vocab 157184, BF16 KV prefilled to 2048 "
           "positions, batch 1, greedy decode at positions 2048..2055",
    "lmhead": "LM-head GEMV + argmax alone: 157184 x 2560 weight N(0,0.02), hidden vectors N(0,1), "
              "3 weight copies rotated so the 256 MB last-level cache cannot serve repeats",
}


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"{name}_traffic.txt")


def stored_traffic(name: str, steps_per_launch: int = 1):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by a plain-copy calibration), or None when the
    summary is missing, was taken on other kernel sources or on launches of
    another number of steps."""
    from memory_bound_gemv_amd.build import source_digest
    path = traffic_file(name)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_digest") != source_digest():
        return None
    if int(fields.get("steps_per_launch", "1")) != steps_per_launch:
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
    KV head (the step's own K/V included; a sliding-window layer only its
    last W positions), 2 bytes (BF16) or 1 (FP8)."""
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
    # a sliding-window layer of window W reads its last W positions
    span = sum(min(pos + 1, cfg.window(li)) if cfg.window(li) > 0 else pos + 1 for li in range(cfg.n_layers))
    kv = span * 2 * cfg.n_kv_heads * d * kv_el
    return w, kv


def window_bytes(cfg, pos: int, k: int, n_distinct: float) -> int:
    """Algorithmic bytes of a k-token verify window of the routed model at
    pos .. pos+k-1 whose union of routed experts has n_distinct members per
    layer on average: every weight once, KV of [0, pos + k)."""
    w, _ = algorithmic_bytes(cfg, pos)
    expert = 3 * cfg.moe_ffn * cfg.hidden * 17 // 32
    w += int(round(cfg.n_layers * (n_distinct - cfg.top_k) * expert))
    kv = (pos + k) * cfg.n_layers * 2 * cfg.n_kv_heads * cfg.head_dim * (1 if cfg.kv_dtype == "fp8" else 2)
    return w + kv


def batch_bytes(cfg, positions, n_distinct: float) -> int:
    """Mean algorithmic bytes of a batch step whose columns sit at the given
    positions (a list of per-step position lists): every weight once (routed
    layers: the union of the columns' experts, n_distinct per layer on
    average) plus each column's own KV."""
    w, _ = algorithmic_bytes(cfg, 0)
    if cfg.is_moe:
        expert = 3 * cfg.moe_ffn * cfg.hidden * 17 // 32
        w += int(round(cfg.n_layers * (n_distinct - cfg.top_k) * expert))
    kv = [sum(algorithmic_bytes(cfg, p)[1] for p in ps) for ps in positions]
    return int(w + sum(kv) / len(kv))


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


def batch_prefill_lens(cfg, n_seqs):
    """Prefill lengths of the batch sequences: sequence b holds
    prefill * (1 - b / (2 n_seqs)) positions (sequence 0 the full prefill)."""
    return [cfg.prefill - (b * cfg.prefill) // (2 * n_seqs) for b in range(n_seqs)]


def build_device_model(cfg, host, dev, k_max=1, n_seqs=1):
    """The workload on the device: weights, prefilled KV cache, context.
    n_seqs > 1: that many sequences on disjoint pages of one pool, prefilled
    to batch_prefill_lens."""
    import torch

    from memory_bound_gemv_amd import _mbg as M
    from memory_bound_gemv_amd.device_model import DeviceModel
    from synth import gen
    pt = gen.page_table(cfg) if n_seqs == 1 else gen.batch_page_table(cfg, n_seqs)
    lens = batch_prefill_lens(cfg, n_seqs)
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
        dm = DeviceModel(cfg, host, pt, lm_fp8=(lm_codes, lm_scales), experts=experts, device=dev, k_max=k_max)
    elif cfg.kv_dtype == "fp8":
        dm = DeviceModel(cfg, host, pt, kv_dtype="fp8", kv_scales=fp8_pow2_scales(cfg, dev), device=dev,
                         k_max=k_max)
    else:
        dm = DeviceModel(cfg, host, pt, device=dev, k_max=k_max)
    for li in range(cfg.n_layers):
        if cfg.kv_dtype == "fp8":
            blk = 1 << 16
            for b, T in enumerate(lens):
                for p0 in range(0, T, blk):
                    n = min(blk, T - p0)
                    dm.kv_write(li, p0, gen.kv_prefill_f32_device(cfg, li, 0, p0, n, dev),
                                gen.kv_prefill_f32_device(cfg, li, 1, p0, n, dev), seq=b)
        else:
            k, v = gen.kv_prefill_bf16(cfg, li)
            for b, T in enumerate(lens):
                dm.prefill_bf16(li, k[:T], v[:T], seq=b)
    dm.init()
    return dm


def build_draft_model(cfg, host, dev, target):
    """A 1-layer early-exit draft for speculative rounds: the target's layer
    0 with its embedding, final norm and LM head (the same device tensors
    for the experts and the FP8 head), its own KV cache prefilled like the
    target's layer 0."""
    from memory_bound_gemv_amd.device_model import DeviceModel
    from synth import gen
    dcfg = cfg.with_(n_layers=1)
    keep = {k: v for k, v in host.items() if not k.startswith("l") or k.startswith("l0.") or k == "lm_head"}
    if cfg.is_moe:
        dm = DeviceModel(dcfg, keep, gen.page_table(dcfg), lm_fp8=(target.lm_codes, target.lm_scales),
                         experts=target.experts[:1], device=dev)
    else:
        dm = DeviceModel(dcfg, keep, gen.page_table(dcfg), device=dev)
    k, v = gen.kv_prefill_bf16(cfg, 0)
    dm.prefill_bf16(0, k, v)
    dm.init()
    return dm


def _threads():
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def cpu_baseline(cfg, host, min_s: float = 10.0, max_steps: int = 200):
    """Time the CPU oracle (float64, as it stands) on a few decode steps of
    the same workload.  One untimed step first converts and caches the
    weights (and, for the routed model, the experts that step routes to);
    the timed steps repeat that step's token and position so that they read
    the same cached weights."""
    from oracle import OracleCache, OracleModel, quantize_fp8_rows
    from synth import gen

    t_prep = time.perf_counter()
    if cfg.is_moe:
        om = OracleModel(cfg, host, experts=lambda l, e, w: gen.expert_mxfp4(cfg, l, e, w),
                         lm_fp8=quantize_fp8_rows(host["lm_head"]))
    else:
        om = OracleModel(cfg, host)
    oc = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    for li in range(cfg.n_layers):
        k, v = gen.kv_prefill_bf16(cfg, li)
        oc.k[li][:cfg.prefill] = k
        oc.v[li][:cfg.prefill] = v
    tok = int(gen.prompt_tokens(cfg, 1)[0])
    om.step(oc, tok, cfg.prefill)
    t_prep = time.perf_counter() - t_prep
    t0 = time.perf_counter()
    steps = 0
    while steps < 2 or (time.perf_counter() - t0 < min_s and steps < max_steps):
        om.step(oc, tok, cfg.prefill)
        steps += 1
    dt = time.perf_counter() - t0
    what = "decode steps" + (" (top-8 of 512 MXFP4 experts + shared per layer, FP8 LM head)" if cfg.is_moe else "")
    return {"value": round(steps / dt, 4), "unit": "tokens/s", "cores": _threads(), "kind": "oracle",
            "sample": (f"{steps} float64 oracle {what} of the same workload, each at position {cfg.prefill} "
                       f"with the same token, after one untimed step ({t_prep:.1f} s including weight "
                       f"conversion{', FP8 LM-head quantisation' if cfg.is_moe else ''}) that cached the weights "
                       f"it reads; {dt:.1f} s timed; host cpu_count {os.cpu_count()}")}


def timed(stream, fn, n):
    """Milliseconds per call of fn() over n back-to-back calls, measured with
    HIP events on the stream the calls are launched on."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def run_decode(args, cfg):
    import numpy as np
    import torch

    from synth import gen

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    host = gen.dense_weights(cfg)
    k_win = 4 if cfg.is_moe and not args.no_verify else 1
    n_batch = args.batch if cfg.kv_dtype == "bf16" else 1
    k_spec = 4 if args.spec and cfg.kv_dtype == "bf16" else 1
    dm = build_device_model(cfg, host, dev, k_max=max(k_win, n_batch, k_spec), n_seqs=n_batch)
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

    wall0 = time.perf_counter()
    ms_per_step = timed(stream, lambda i: dm.step(buf, pos_of(args.warmup + i), logits, buf), args.steps)
    wall = time.perf_counter() - wall0
    st = dm.status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    tok_s = 1e3 / ms_per_step

    wbytes, _ = algorithmic_bytes(cfg, 0)
    kv_avg = float(np.mean([algorithmic_bytes(cfg, pos_of(args.warmup + i))[1] for i in range(args.steps)]))
    step_bytes = wbytes + kv_avg
    single = {"tokens_s": round(tok_s, 2), "ms_per_step": round(ms_per_step, 4), "launches_per_token": 1}
    launches_per_token = 1.0
    G = min(args.multi_step, cfg.n_decode, args.steps)
    if G > 1:
        # G greedy steps per launch (positions prefill .. prefill + G - 1);
        # each launch reads its first token on the device from the previous
        # launch's last argmax (two token buffers used in turn).  Exactly
        # args.steps steps are timed: the last launch takes the remainder.
        tk = [torch.zeros(G, dtype=torch.int32, device=dev) for _ in range(2)]
        tk[1][G - 1] = int(gen.prompt_tokens(cfg, 1)[0])
        sizes = [G] * (args.steps // G) + ([args.steps % G] if args.steps % G else [])
        last = [G - 1]   # index of the previous launch's last argmax in its buffer

        def launch(i, g=G):
            dm.steps(tk[(i + 1) % 2][last[0]:], g, cfg.prefill, None, tk[i % 2])
            last[0] = g - 1

        for i in range(max(1, args.warmup // G)):
            launch(i)
        ms_total = timed(stream, lambda i: launch(i, sizes[i]), len(sizes)) * len(sizes)
        if dm.status() != 0:
            raise RuntimeError("device status after the multi-step launches")
        ms_per_step = ms_total / args.steps
        tok_s = 1e3 / ms_per_step
        launches_per_token = len(sizes) / args.steps
        kv_avg = float(np.mean([algorithmic_bytes(cfg, cfg.prefill + i)[1] for s_ in sizes for i in range(s_)]))
        step_bytes = wbytes + kv_avg
    spl = max(G, 1)   # steps per (full) launch of the timed configuration
    achieved = step_bytes / (ms_per_step / 1e3) / 1e9
    traffic = stored_traffic(f"step_kernel_{args.workload}", spl)

    out = {
        "metric": METRIC,
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
            "weight_dtype": "bf16 attention/router + mxfp4 experts + fp8 lm head" if cfg.is_moe else "bf16",
            "kv_dtype": cfg.kv_dtype, "accumulate": "fp32",
            "global_batch": 1, "seq_len": cfg.prefill, "parallelism": "none (1 GPU)",
            "kernel": info.variant.decode(), "grid": info.grid, "launches_per_step": round(launches_per_token, 4),
            "steps_per_launch": spl,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "bytes_per_step": {"weights": wbytes, "kv_avg": round(kv_avg), "total": round(step_bytes)},
        "ms_per_launch": round(ms_per_step * spl, 4),
        "single_step_launches": single,
        "bound_tokens_s": round(PEAK_HBM_GBS * 1e9 / step_bytes, 1),
        "wall_tokens_s": round(args.steps / wall, 2),
        "setup_s": round(t_gen, 1),
    }
    if traffic is not None:
        # beta: bytes moved per algorithmic weight byte (the KV history is
        # counted as read once); traffic covers the steps of one launch
        beta = (traffic / spl - kv_avg) / wbytes
        out["beta"] = round(beta, 4)
        out["bound_tokens_s_measured_beta"] = round(PEAK_HBM_GBS * 1e9 / (beta * wbytes + kv_avg), 1)

    if k_win == 4:
        # the 4-token verify window over the tokens of four steps, at the
        # first decode position (rewriting the same four cache positions)
        win = torch.tensor([int(t) for t in gen.prompt_tokens(cfg, 4)], dtype=torch.int32, device=dev)
        wl = torch.empty((4, cfg.vocab), dtype=torch.float32, device=dev)
        wa = torch.zeros(4, dtype=torch.int32, device=dev)
        from memory_bound_gemv_amd import _mbg as M
        ms_path = {}
        for path in (M.MBG_PATH_FMA, M.MBG_PATH_MFMA):
            M.mbg_set_verify_path(dm.ctx, path)
            for _ in range(3):
                dm.verify(win, cfg.prefill, wl, wa)
            ms_path[path] = timed(stream, lambda i: dm.verify(win, cfg.prefill, wl, wa), max(5, args.steps // 4))
            if dm.status() != 0:
                raise RuntimeError("device status after the verify windows")
        best = min(ms_path, key=ms_path.get)
        M.mbg_set_verify_path(dm.ctx, best)
        dm.verify(win, cfg.prefill, wl, wa)
        ms_win = ms_path[best]
        distinct = []
        for li in range(cfg.n_layers):
            idx, _ = dm.routing(li)
            distinct.append(len(np.unique(idx)))
        nd = float(np.mean(distinct))
        wb = window_bytes(cfg, cfg.prefill, 4, nd)
        out["verify_window"] = {
            "k": 4, "ms_per_window": round(ms_win, 4), "tokens_s": round(4e3 / ms_win, 1),
            "window_over_step": round(ms_win / ms_per_step, 3), "distinct_experts_per_layer": round(nd, 2),
            "bytes_per_window": wb, "achieved_GBs": round(wb / (ms_win / 1e3) / 1e9, 1),
            "path": "mfma" if best == M.MBG_PATH_MFMA else "fma",
            "ms_per_window_fma": round(ms_path[M.MBG_PATH_FMA], 4),
            "ms_per_window_mfma": round(ms_path[M.MBG_PATH_MFMA], 4),
        }

    if args.spec and cfg.kv_dtype == "bf16" and dm.k_max >= 4:
        # speculative rounds (k = 4): 1-layer early-exit draft, verify and
        # on-device acceptance, two launches per round; one round from a
        # fixed state repeated (the workload's position budget holds only a
        # few rounds), its acceptance read back
        ddm = build_draft_model(cfg, host, dev, dm)
        s0 = torch.zeros(12, dtype=torch.int32, device=dev)
        s0[0] = cfg.prefill
        s0[4] = int(gen.prompt_tokens(cfg, 1)[0])
        s1 = torch.zeros_like(s0)
        emit = torch.zeros(16, dtype=torch.int32, device=dev)
        tk4 = torch.zeros(4, dtype=torch.int32, device=dev)
        tk4[0] = int(s0[4].item())
        am4 = torch.zeros(4, dtype=torch.int32, device=dev)
        for _ in range(3):
            dm.spec_round(ddm, 4, s0, s1, emit)
        ms_round = timed(stream, lambda i: dm.spec_round(ddm, 4, s0, s1, emit), max(8, args.steps // 8))
        ms_draft = timed(stream, lambda i: ddm.steps(tk4, 4, cfg.prefill, None, am4), max(8, args.steps // 8))
        if dm.status() != 0 or ddm.status() != 0:
            raise RuntimeError("device status after the speculative rounds")
        m = int(s1[2].item())
        out["spec_round"] = {
            "k": 4, "draft": "1 layer (the target's layer 0, embedding, final norm and LM head)",
            "ms_per_round": round(ms_round, 4), "ms_draft_4_steps": round(ms_draft, 4),
            "accepted_this_round": m, "tokens_s_at_this_acceptance": round((m + 1) * 1e3 / ms_round, 1),
            "tokens_s_full_acceptance": round(4e3 / ms_round, 1),
            "note": "random weights: acceptance measures nothing; the round's cost is what is measured",
        }
        ddm.close()

    if n_batch > 1:
        # n_batch independent sequences per step, each at its own position
        # (sequence b from batch_prefill_lens(b), positions cycled over
        # n_decode slots like the single-sequence steps)
        lens = batch_prefill_lens(cfg, n_batch)
        seqs = list(range(n_batch))
        btok = torch.tensor([int(t) for t in gen.prompt_tokens(cfg, n_batch)], dtype=torch.int32, device=dev)
        bam = torch.zeros(n_batch, dtype=torch.int32, device=dev)
        bpos = lambda i: [L + (i % n_slots) for L in lens]
        for i in range(max(3, args.warmup // 4)):
            dm.batch(btok, seqs, bpos(i), None, bam)
        ms_b = timed(stream, lambda i: dm.batch(btok, seqs, bpos(i), None, bam), max(8, args.steps // 4))
        if dm.status() != 0:
            raise RuntimeError("device status after the batch steps")
        nd = 1.0
        if cfg.is_moe:
            dm.batch(btok, seqs, bpos(0), None, bam)
            nd = float(np.mean([len(np.unique(dm.routing(li)[0][:n_batch])) for li in range(cfg.n_layers)]))
        bb = batch_bytes(cfg, [bpos(i) for i in range(n_slots)], nd)
        out["batch"] = {
            "n": n_batch, "prefill_lens": lens, "ms_per_step": round(ms_b, 4),
            "tokens_s": round(n_batch * 1e3 / ms_b, 1),
            "tokens_s_over_batch1": round(n_batch * 1e3 / ms_b / out["value"], 3),
            "distinct_experts_per_layer": round(nd, 2) if cfg.is_moe else None,
            "bytes_per_step": bb, "achieved_GBs": round(bb / (ms_b / 1e3) / 1e9, 1),
            "frac": round(bb / (ms_b / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
        }

    if args.trace:
        from memory_bound_gemv_amd import _mbg as M
        M.mbg_set_trace(dm.ctx, True)
        dm.step(buf, pos_of(args.warmup + args.steps), logits, buf)
        rec = M.mbg_read_trace(dm.ctx, info.n_tasks)
        M.mbg_set_trace(dm.ctx, False)
        np.save(args.trace, rec)
        np.save(args.trace.replace(".npy", "_meta.npy"),
                np.array([info.clock_khz, info.grid, cfg.n_layers], dtype=np.int64))

    copy_probe(args, dev)
    if not args.no_cpu_baseline and cfg.kv_dtype == "bf16":
        out["cpu_baseline"] = cpu_baseline(cfg, host)
    dm.close()
    return out


def copy_probe(args, dev):
    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib * 1024 * 1024 // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()


def run_lmhead(args, cfg):
    """The LM-head GEMV + argmax alone, BF16 or FP8 rows, k columns."""
    import numpy as np
    import torch

    from memory_bound_gemv_amd import _mbg as M
    from synth import gen

    dev = torch.device("cuda:0")
    V, H, k = cfg.vocab, cfg.hidden, args.k
    stream = torch.cuda.current_stream(dev)
    w = gen.lm_head_bf16(cfg)
    wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(dev)
    copies = []
    for c in range(3):
        if args.lm_dtype == "fp8":
            codes = torch.empty((V, H), dtype=torch.uint8, device=dev)
            scales = torch.empty(V, dtype=torch.float32, device=dev)
            M.mbg_quantize_fp8_rows(wd, V, H, codes, scales, stream.cuda_stream)
            copies.append((M.make_tensor(codes, "fp8", V, H, scale=scales), codes, scales))
        else:
            t = wd.clone()
            copies.append((M.make_tensor(t, "bf16", V, H), t))
    del wd
    x = torch.from_numpy(gen.lm_head_inputs(cfg, k)).to(dev)
    logits = torch.empty((k, V), dtype=torch.float32, device=dev)
    amax = torch.zeros(k, dtype=torch.int32, device=dev)
    nbytes = M.mbg_lm_head_workspace_size(k)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    call = lambda i: M.mbg_lm_head(copies[i % 3][0], x, k, logits, amax, ws, nbytes, stream.cuda_stream)
    for i in range(args.warmup):
        call(i)
    ms = timed(stream, call, args.steps)
    wbytes = V * H * (1 if args.lm_dtype == "fp8" else 2) + (4 * V if args.lm_dtype == "fp8" else 0)
    achieved = wbytes / (ms / 1e3) / 1e9
    name = f"lm_head_kernel_{args.lm_dtype}_k{k}"
    copy_probe(args, dev)
    return {
        "metric": "LM-head GEMV + argmax: calls/s and achieved HBM GB/s (MBU % of peak) on 1 MI355X",
        "value": round(1e3 / ms, 1), "unit": "calls/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic",
        "config": {"workload": WORKLOADS["lmhead"], "weight_dtype": args.lm_dtype, "columns": k},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": stored_traffic(name)},
        "bytes_per_call": wbytes,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="moe", choices=["moe", "dense2b", "longctx", "longctx_swa", "lmhead"],
                    help="moe (default: the routed 42-layer model), dense2b, longctx (FP8 KV at 200K "
                         "positions), longctx_swa (the same with sliding-window layers) or lmhead (the "
                         "LM-head GEMV alone)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="moe: skip the 4-token verify-window timing")
    ap.add_argument("--no-spec", dest="spec", action="store_false",
                    help="skip the speculative-round timing (BF16-KV workloads)")
    ap.add_argument("--batch", type=int, default=4,
                    help="also time steps of this many independent sequences (BF16-KV workloads; 1: skip)")
    ap.add_argument("--multi-step", type=int, default=8,
                    help="steps per launch of the headline timing (1: single-step launches only); "
                         "single-step launches are timed beside it")
    ap.add_argument("--lm-dtype", default="fp8", choices=["bf16", "fp8"], help="lmhead: weight format")
    ap.add_argument("--k", type=int, default=1, help="lmhead: activation columns (1..4)")
    ap.add_argument("--trace", default="",
                    help="after the timed region, run one traced step and save its per-task stamps (.npy)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    from synth import CONFIGS
    cfg = CONFIGS[args.workload]
    out = run_lmhead(args, cfg) if args.workload == "lmhead" else run_decode(args, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
