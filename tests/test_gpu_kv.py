"""GPU tests of the KV cache in its stored formats.

* mbg_kv_write (the prefill entry point) rounds float32 K/V into the paged
  pool bit-exactly as the oracle's codecs do (BF16 nearest-even; FP8 E4M3FN
  of x / scale, nearest-even, saturating), pages shuffled.
* The dense 2B decoder with an FP8 cache (per-head power-of-two scales, not
  1.0) matches the oracle, teacher-forced.
* The long-context workload itself: FP8 cache prefilled to 200,000 positions
  under a shuffled page table, one full decode step against the oracle.
"""
import numpy as np
import pytest

from gpu_util import build_dense, check_argmax, compare_logits, say
from oracle import OracleCache, codecs
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _special_f32(rng, n):
    """Random float32 values plus the cases rounding must get right."""
    x = np.concatenate([
        rng.standard_normal(n).astype(np.float32) * 40,
        rng.standard_normal(n // 4).astype(np.float32) * 1e-3,            # FP8 subnormal range
        (rng.integers(0, 2**32, n // 4, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        # FP8 ties: midpoints between neighbouring codes, and values around 448
        np.array([0.5 * (1 + 1.125), 0.5 * (1.125 + 1.25), 2.0**-9 * 0.5, 2.0**-9 * 1.5, 2.0**-9 * 2.5,
                  416.0, 432.0, 440.0, 447.9, 448.0, 460.0, 464.0, 465.0, 1e30, np.inf, -np.inf, np.nan,
                  -0.0, 0.0, -2.0**-10, 2.0**-10], dtype=np.float32),
    ])
    return x[np.isfinite(x) | np.isinf(x) | np.isnan(x)]


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_kv_write_bitexact(kv_dtype):
    from memory_bound_gemv_amd.device_model import DeviceModel
    cfg = CONFIGS["tiny"].with_(page_size=16, kv_dtype=kv_dtype)
    say("kv_write", kv_dtype)
    host = gen.dense_weights(cfg)
    pt = gen.page_table(cfg, True)
    L, Hkv, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    scales = np.array([[[2.0**-6, 0.75], [3.0, 1.0]]] * L, dtype=np.float32)  # [L][Hkv][2]
    dm = DeviceModel(cfg, host, pt, kv_dtype=kv_dtype, kv_scales=scales if kv_dtype == "fp8" else None)
    rng = np.random.default_rng(11)
    T = cfg.max_pos
    oc = OracleCache(L, T, Hkv, d, kv_dtype)
    if kv_dtype == "fp8":
        oc.scales = scales
    inputs = []
    for li in range(L):
        vals = _special_f32(rng, 2 * T * Hkv * d)
        vals = np.resize(rng.permutation(vals), (2, T, Hkv, d)).astype(np.float32)
        k, v = vals[0], vals[1]
        # two writes that together cover [0, T): a ragged split across pages
        cut = 21
        for p0, p1 in ((0, cut), (cut, T)):
            dm.kv_write(li, p0, torch.from_numpy(np.ascontiguousarray(k[p0:p1])).cuda(),
                        torch.from_numpy(np.ascontiguousarray(v[p0:p1])).cuda())
        oc.prefill_f32(li, 0, k, v)
        inputs.append((k, v))
    torch.cuda.synchronize()
    for li in range(L):
        gk, gv = dm.cache_logical(li, T)
        for name, g, r, x in (("K", gk, oc.k[li], inputs[li][0]), ("V", gv, oc.v[li], inputs[li][1])):
            if kv_dtype == "bf16":
                # NaN has no single BF16 pattern: both sides must give a NaN of the same sign
                nan = np.isnan(x)
                assert np.all((g[nan] & 0x7FFF) > 0x7F80) and np.all((g[nan] >> 15) == (r[nan] >> 15))
                g, r = g[~nan], r[~nan]
            assert np.array_equal(g, r), f"layer {li} {name}: {np.sum(g != r)} codes differ"
    # the direct codec agrees with the bulk one used above
    if kv_dtype == "fp8":
        y = (k / scales[0, :, 0][None, :, None]).astype(np.float32)
        assert np.array_equal(codecs.f32_to_fp8e4m3(y), oc.k[L - 1])


def _teacher_forced(dm, om, oc, cfg, n_steps, what):
    toks = gen.prompt_tokens(cfg, n_steps)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    nxt = int(toks[0])
    graded = 0
    for i in range(n_steps):
        pos = cfg.prefill + i
        tok.fill_(nxt)
        dm.step(tok, pos, logits, amax)
        torch.cuda.synchronize()
        g = logits.cpu().numpy()
        ref = om.step(oc, nxt, pos)
        ma, rel = compare_logits(g, ref, what=f"{what} step {i} pos {pos}")
        say(f"{what} step {i}: max abs {ma:.2e} rel L2 {rel:.2e}")
        a = int(amax.item())
        graded += check_argmax(a, g, ref, what=f"{what} step {i}")
        nxt = a
    assert dm.status() == 0
    return graded


def test_dense2b_fp8_kv_steps():
    """Dense 2B with an FP8 cache prefilled to 4096 positions, shuffled pages."""
    cfg = CONFIGS["dense2b"].with_(kv_dtype="fp8", shuffled_pages=True)
    say("dense2b fp8 kv build")
    dm, om, oc = build_dense(cfg)
    info = dm.info()
    assert info.kv_dtype == 2 and b"fp8kv" in info.variant
    sc = oc.scales
    assert np.all(sc != 1.0), "the per-head scales must not be the 1.0 fallback"
    say("scales", np.unique(sc))
    _teacher_forced(dm, om, oc, cfg, 3, "dense2b-fp8kv")


@pytest.mark.parametrize("kv,k", [("bf16", 4), ("fp8", 3), ("fp8", 4)])
def test_verify_window_streamed_history(kv, k):
    """A verify window whose split histories are longer than the attention
    ring (24,000 positions: over 512 per split), so the history streams
    through LDS instead of staying resident there.  Over the FP8 cache the
    window's columns fold each history chunk as it passes (all k at once, or
    two pairs for k = 4, the second pair streaming the history again); over
    the BF16 cache each column streams it in turn.  Every column is compared
    with the oracle."""
    cfg = CONFIGS["dense2b"].with_(name="dense2b", kv_dtype=kv, prefill=24000, n_decode=8,
                                   shuffled_pages=True)
    say("streamed-history verify", kv, k)
    dm, om, oc = build_dense(cfg)
    info = dm.info()
    assert (cfg.prefill + info.attn_splits - 1) // info.attn_splits > 512, "splits must not fit the ring"
    p0 = cfg.prefill
    toks = [int(t) for t in gen.prompt_tokens(cfg, k)]
    win = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty((k, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(k, dtype=torch.int32, device="cuda")
    dm.verify(win, p0, logits, am)
    torch.cuda.synchronize()
    g = logits.cpu().numpy()
    amh = am.cpu().numpy()
    ref = om.verify(oc, toks, p0)
    for j in range(k):
        compare_logits(g[j], ref[j], what=f"{kv} streamed verify col {j}")
        check_argmax(int(amh[j]), g[j], ref[j], what=f"{kv} streamed verify col {j}")
    assert dm.status() == 0


@pytest.mark.parametrize("k", [2, 4])
def test_fp8_kv_verify_window(k):
    """Verify window on the FP8-cache kernel: k tokens in one launch against
    the oracle (token j sees [0, pos + j], the window's own FP8 K/V included)
    and against k single steps of a second context."""
    cfg = CONFIGS["dense2b"].with_(name="dense2b", kv_dtype="fp8", prefill=1000, n_decode=8,
                                   shuffled_pages=True)
    say("fp8 kv verify", k)
    host = gen.dense_weights(cfg)
    dm, om, oc = build_dense(cfg, host=host)
    p0 = cfg.prefill
    toks = [int(t) for t in gen.prompt_tokens(cfg, k)]
    win = torch.tensor(toks, dtype=torch.int32, device="cuda")
    logits = torch.empty((k, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(k, dtype=torch.int32, device="cuda")
    dm.verify(win, p0, logits, am)
    torch.cuda.synchronize()
    g = logits.cpu().numpy()
    amh = am.cpu().numpy()
    ref = om.verify(oc, toks, p0)
    for j in range(k):
        compare_logits(g[j], ref[j], what=f"fp8 verify col {j}")
        check_argmax(int(amh[j]), g[j], ref[j], what=f"fp8 verify col {j}")
    assert dm.status() == 0
    dm2, _, _ = build_dense(cfg, host=host, kv_scales=oc.scales)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    l1 = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    a1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    for j in range(k):
        tok.fill_(toks[j])
        dm2.step(tok, p0 + j, l1, a1)
        d = float(np.max(np.abs(l1.cpu().numpy() - g[j])))
        assert d < 2e-3, f"verify col {j} vs step: max abs {d}"
    assert dm2.status() == 0


@pytest.mark.timeout(1500)
def test_longctx_fp8_kv_200k():
    """The long-context workload: FP8 cache prefilled to 200,000 positions in
    64-token pages under a shuffled page table; two greedy decode steps at
    200,000 and 200,001 (the second reads the FP8 K/V the kernel wrote in
    the first)."""
    cfg = CONFIGS["longctx"]
    assert cfg.prefill == 200000 and cfg.kv_dtype == "fp8" and cfg.shuffled_pages
    say("longctx build (prefill 200000, fp8)")
    dm, om, oc = build_dense(cfg)
    pt = dm.page_table_host
    assert not np.array_equal(pt, np.arange(pt.size))
    say("longctx info", dm.info().grid, dm.info().attn_splits, dm.info().variant)
    _teacher_forced(dm, om, oc, cfg, 2, "longctx")
    # the cache entries the kernel wrote at 200,000 and 200,001 equal the
    # oracle's codes, up to one FP8 step where the binary32 values straddle
    # a rounding boundary
    for li in (0, cfg.n_layers - 1):
        P = cfg.page_size
        for pos in (cfg.prefill, cfg.prefill + 1):
            page = int(dm.page_table_host[pos // P])
            for which, ref in ((0, oc.k[li][pos]), (1, oc.v[li][pos])):
                got = dm.pool[li, page, which, :, pos % P, :].cpu().numpy()
                a = codecs.fp8e4m3_to_f64(got)
                b = codecs.fp8e4m3_to_f64(ref)
                frac = float(np.mean(got == ref))
                say(f"longctx cache layer {li} pos {pos} kv {which}: bit-equal {frac:.4f}")
                assert frac > 0.95
                assert np.all(np.abs(a - b) <= 2.0 ** -3 * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -9)
