"""GPU parity of the routed (MoE) decode path against the CPU oracle.

* MXFP4 GEMV through the C-ABI: a one-hot input returns each dequantised
  weight exactly (every E2M1 code, every E8M0 scale with finite products), random
  inputs match within tolerance.
* A small routed model with the compiled MoE shape (2 layers, 64 experts,
  top-8 plus one shared expert, FP8 LM head): teacher-forced steps, routing
  decisions and weights, and a 4-token verify window (the union of the
  tokens' experts) against both the oracle and the single steps.
* The full routed workload: 42 layers, 512 experts, vocab 157,184, KV
  prefilled to 2048 positions; four steps, then the verify window over the
  same four tokens.
"""
import numpy as np
import pytest

from gpu_util import LOGIT_REL_L2_MXFP4, build_moe, check_argmax, compare_logits, say
from oracle import codecs
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROUTE_GAP = 1e-2     # routing graded exactly where the 8th/9th logit gap exceeds this


def _M():
    from memory_bound_gemv_amd import _mbg
    return _mbg


def _gemv_mxfp4(codes, scales, x):
    M = _M()
    V, half = codes.shape
    H = 2 * half
    k = x.shape[0]
    cd = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
    sd = torch.from_numpy(np.ascontiguousarray(scales)).cuda()
    xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    logits = torch.empty((k, V), dtype=torch.float32, device="cuda")
    amax = torch.zeros(k, dtype=torch.int32, device="cuda")
    nbytes = M.mbg_lm_head_workspace_size(k)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    M.mbg_lm_head(M.make_tensor(cd, "mxfp4", V, H, scale=sd), xd, k, logits, amax, ws, nbytes,
                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), amax.cpu().numpy()


def test_mxfp4_onehot_dequant_is_exact():
    """x = e_j returns column j of the dequantised matrix bit for bit, over
    every E2M1 code and every E8M0 scale byte whose products stay finite in
    binary32 (0 .. 252: 6 x 2^125 is the largest; from 253 on, 6 x 2^126
    overflows and the other columns' inf x 0 would make the sum NaN).  The
    smallest scales give binary32 subnormals, which must not be flushed."""
    V, H = 512, 256
    rng = np.random.default_rng(21)
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = np.resize(np.arange(253, dtype=np.uint8), V * H // 32).reshape(V, H // 32)
    scales = scales[rng.permutation(V)]
    ref = codecs.mxfp4_to_f64(codes, scales)
    cols = [0, 1, 31, 32, 100, 255]
    assert len(np.unique(codes & 0xF)) == 16
    for j0 in range(0, len(cols), 4):
        js = cols[j0:j0 + 4]
        x = np.zeros((len(js), H), dtype=np.float32)
        for c, j in enumerate(js):
            x[c, j] = 1.0
        got, _ = _gemv_mxfp4(codes, scales, x)
        for c, j in enumerate(js):
            want = ref[:, j].astype(np.float32)
            assert np.array_equal(got[c], want), f"column {j}: {np.sum(got[c] != want)} values differ"


@pytest.mark.parametrize("k", [1, 4])
def test_mxfp4_gemv_random(k):
    V, H = 1000, 2560
    rng = np.random.default_rng(30 + k)
    codes = rng.integers(0, 256, (V, H // 2), dtype=np.uint8)
    scales = rng.integers(120, 123, (V, H // 32), dtype=np.uint8)
    x = rng.standard_normal((k, H)).astype(np.float32)
    got, idx = _gemv_mxfp4(codes, scales, x)
    ref = x.astype(np.float64) @ codecs.mxfp4_to_f64(codes, scales).T
    for c in range(k):
        compare_logits(got[c], ref[c], rel_tol=LOGIT_REL_L2_MXFP4, what=f"mxfp4 col {c}")
        check_argmax(int(idx[c]), got[c], ref[c], what=f"mxfp4 col {c}")


def _check_routing(dm, om, cfg, what, col=0):
    """GPU routing of the last call (column `col`) against the oracle's last step."""
    graded = 0
    for li in range(cfg.n_layers):
        idx, w = dm.routing(li)
        sel, wts, r = om.last_routing[li]
        r32 = np.sort(np.asarray(r, dtype=np.float32))[::-1]
        if r32[cfg.top_k - 1] - r32[cfg.top_k] > ROUTE_GAP:
            assert list(idx[col]) == [int(e) for e in sel], f"{what} layer {li}: {idx[col]} vs {sel}"
            assert np.allclose(w[col], wts, atol=2e-3), f"{what} layer {li}: weights {w[col]} vs {wts}"
            graded += 1
        assert abs(float(np.sum(w[col])) - 1.0) < 1e-5
    return graded


def _steps(dm, om, oc, cfg, p0, toks, what):
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs, routed = [], 0
    for i, t in enumerate(toks):
        tok.fill_(int(t))
        dm.step(tok, p0 + i, logits, amax)
        torch.cuda.synchronize()
        g = logits.cpu().numpy()
        ref = om.step(oc, int(t), p0 + i)
        ma, rel = compare_logits(g, ref, rel_tol=LOGIT_REL_L2_MXFP4, what=f"{what} step {i}")
        routed += _check_routing(dm, om, cfg, f"{what} step {i}")
        check_argmax(int(amax.item()), g, ref, what=f"{what} step {i}")
        say(f"{what} step {i} pos {p0 + i}: max abs {ma:.2e} rel L2 {rel:.2e}")
        outs.append((g.copy(), ref))
    assert dm.status() == 0
    return outs, routed


def _verify(dm, cfg, p0, toks, steps, what, path=None):
    k = len(toks)
    if path is not None:
        _M().mbg_set_verify_path(dm.ctx, path)
        assert dm.info().verify_path == path
    win = torch.from_numpy(np.asarray(toks, dtype=np.int32)).cuda()
    logits = torch.empty((k, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(k, dtype=torch.int32, device="cuda")
    dm.verify(win, p0, logits, am)
    torch.cuda.synchronize()
    g = logits.cpu().numpy()
    amh = am.cpu().numpy()
    idx, _ = dm.routing(0)
    say(f"{what}: verify routing layer 0 union {len(np.unique(idx))} experts")
    for j in range(k):
        step_g, ref = steps[j]
        compare_logits(g[j], ref, rel_tol=LOGIT_REL_L2_MXFP4, what=f"{what} verify col {j} vs oracle")
        d = float(np.max(np.abs(g[j] - step_g)))
        assert d < 2e-3, f"{what} verify col {j} vs step: max abs {d}"
        check_argmax(int(amh[j]), g[j], ref, what=f"{what} verify col {j}")
    assert dm.status() == 0


MOE_SMALL = CONFIGS["moe"].with_(name="moe_small", n_layers=2, n_experts=64, vocab=4096, prefill=256,
                                 n_decode=8)


def test_moe_small_steps_and_verify():
    cfg = MOE_SMALL
    say("moe_small build")
    dm, om, oc = build_moe(cfg)
    info = dm.info()
    assert info.expert_dtype == 3 and info.lm_dtype == 2 and info.variant.decode().endswith("moe")
    toks = gen.prompt_tokens(cfg, 4)
    steps, routed = _steps(dm, om, oc, cfg, cfg.prefill, toks, "moe_small")
    say("moe_small graded routing decisions", routed)
    assert routed >= 4
    _verify(dm, cfg, cfg.prefill, toks, steps, "moe_small")
    # a 2-token window too (union smaller than one expert-down pass)
    dm2, _, _ = build_moe(cfg)
    _steps_only = []
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    am = torch.zeros(1, dtype=torch.int32, device="cuda")
    lg = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    for i in range(2):
        tok.fill_(int(toks[i]))
        dm2.step(tok, cfg.prefill + i, lg, am)
        _steps_only.append((lg.cpu().numpy().copy(), steps[i][1]))
    _verify(dm2, cfg, cfg.prefill, toks[:2], _steps_only, "moe_small k=2")


@pytest.mark.parametrize("top_k,n_shared", [(4, 2), (2, 0)])
def test_moe_small_other_topk_and_shared(top_k, n_shared):
    """Top-k and the shared-expert count are run-time: four routed experts
    plus two shared ones, and two routed with none, on the compiled routed
    shape; steps (logits, argmax, graded routing decisions and weights) and
    a 4-token verify window against the oracle and the steps."""
    cfg = MOE_SMALL.with_(name=f"moe_small_k{top_k}s{n_shared}", top_k=top_k, n_shared=n_shared)
    say(cfg.name, "build")
    dm, om, oc = build_moe(cfg)
    toks = gen.prompt_tokens(cfg, 4)
    steps, routed = _steps(dm, om, oc, cfg, cfg.prefill, toks, cfg.name)
    say(cfg.name, "graded routing decisions", routed)
    assert routed >= 4
    _verify(dm, cfg, cfg.prefill, toks, steps, cfg.name)


def test_moe_small_routing_ties():
    """Equal router logits: every router row is zero except experts 20, 30,
    31 and 45, and the last three are one row, so each decision holds a tie
    of three (two experts in one lane of the selection, one in another) and
    one of the remaining zeros; the top-k takes equal values in index order
    (the oracle's rule).  Picks and weights match the oracle exactly wherever
    the three distinct values (a, b, 0) are apart, and a 4-token verify
    window (one wave per column) matches its single steps."""
    cfg = MOE_SMALL
    host = gen.dense_weights(cfg)
    for li in range(cfg.n_layers):
        w = np.zeros_like(host[f"l{li}.w_router"])
        w[20] = host[f"l{li}.w_router"][20]
        w[[30, 31, 45]] = host[f"l{li}.w_router"][30]
        host[f"l{li}.w_router"] = w
    say("moe_small ties build")
    dm, om, oc = build_moe(cfg, host=host)
    toks = gen.prompt_tokens(cfg, 4)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    steps, graded, zeros_picked = [], 0, 0
    for i, t in enumerate(toks):
        tok.fill_(int(t))
        dm.step(tok, cfg.prefill + i, logits, amax)
        torch.cuda.synchronize()
        g = logits.cpu().numpy()
        ref = om.step(oc, int(t), cfg.prefill + i)
        compare_logits(g, ref, rel_tol=LOGIT_REL_L2_MXFP4, what=f"ties step {i}")
        check_argmax(int(amax.item()), g, ref, what=f"ties step {i}")
        for li in range(cfg.n_layers):
            idx, wts = dm.routing(li)
            sel, owts, r = om.last_routing[li]
            a, b = float(r[20]), float(r[30])
            assert r[30] == r[31] == r[45] and np.count_nonzero(r) <= 4
            if min(abs(a), abs(b), abs(a - b)) > 1e-3:
                assert list(idx[0]) == [int(e) for e in sel], f"layer {li} step {i}: {idx[0]} vs {sel}"
                assert np.allclose(wts[0], owts, atol=2e-3), f"layer {li} step {i}: {wts[0]} vs {owts}"
                graded += 1
            zeros_picked += int(np.sum(idx[0] < 8))
        steps.append((g.copy(), ref))
    say("ties graded", graded, "of", 4 * cfg.n_layers, "zero-logit picks", zeros_picked)
    assert graded >= 2 * cfg.n_layers and zeros_picked > 0
    _verify(dm, cfg, cfg.prefill, toks, steps, "moe_small ties")
    assert dm.status() == 0


@pytest.mark.timeout(1500)
def test_moe_full_step_and_verify():
    """The routed workload at full size: all 8 decode steps at 2048..2055,
    then the 4-token verify window at 2048 over the first four tokens."""
    cfg = CONFIGS["moe"]
    assert cfg.n_layers == 42 and cfg.n_experts == 512 and cfg.vocab == 157184 and cfg.prefill == 2048
    say("moe full build")
    dm, om, oc = build_moe(cfg, cache_experts=False)
    info = dm.info()
    say("moe full info", info.grid, info.attn_splits, info.variant, info.weight_bytes_per_step)
    toks = gen.prompt_tokens(cfg, cfg.n_decode)
    steps, routed = _steps(dm, om, oc, cfg, cfg.prefill, toks, "moe")
    say("moe graded routing decisions", routed, "of", cfg.n_decode * cfg.n_layers)
    assert routed >= 8 * 42 // 2
    _verify(dm, cfg, cfg.prefill, toks[:4], steps[:4], "moe")
    # the matrix-core expert gate/up path on the same window
    _verify(dm, cfg, cfg.prefill, toks[:4], steps[:4], "moe mfma", path=_M().MBG_PATH_MFMA)


def test_moe_small_multi_step_launch():
    """Routed model: 6 greedy steps in one launch equal 6 single-step
    launches bit for bit (routing, expert phases and KV across steps) and
    match the oracle teacher-forced with the GPU's tokens."""
    from test_gpu_decode import _multi_vs_single
    cfg = MOE_SMALL
    _multi_vs_single(cfg, gen.dense_weights(cfg), build_moe, cfg.prefill, 6, "moe_small multi-step",
                     rel_tol=LOGIT_REL_L2_MXFP4)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_moe_small_verify_mfma(k):
    """Verify window with the expert gate/up rows on the matrix cores (BF16
    hi + lo activations): against the oracle and against k single steps,
    and close to the FMA path's window."""
    M = _M()
    cfg = MOE_SMALL
    host = gen.dense_weights(cfg)
    toks = gen.prompt_tokens(cfg, k)
    dm, om, oc = build_moe(cfg, host=host)
    steps, _ = _steps(dm, om, oc, cfg, cfg.prefill, toks, f"moe_small k={k}")
    win = torch.from_numpy(np.asarray(toks, dtype=np.int32)).cuda()
    outs = {}
    for path in (M.MBG_PATH_FMA, M.MBG_PATH_MFMA):
        M.mbg_set_verify_path(dm.ctx, path)
        logits = torch.empty((k, cfg.vocab), dtype=torch.float32, device="cuda")
        am = torch.zeros(k, dtype=torch.int32, device="cuda")
        dm.verify(win, cfg.prefill, logits, am)
        torch.cuda.synchronize()
        outs[path] = (logits.cpu().numpy(), am.cpu().numpy())
    assert dm.status() == 0
    g, amh = outs[M.MBG_PATH_MFMA]
    for j in range(k):
        step_g, ref = steps[j]
        compare_logits(g[j], ref, rel_tol=LOGIT_REL_L2_MXFP4, what=f"mfma verify col {j} vs oracle")
        d = float(np.max(np.abs(g[j] - step_g)))
        assert d < 2e-3, f"mfma verify col {j} vs step: max abs {d}"
        d2 = float(np.max(np.abs(g[j] - outs[M.MBG_PATH_FMA][0][j])))
        assert d2 < 2e-3, f"mfma vs fma col {j}: max abs {d2}"
        check_argmax(int(amh[j]), g[j], ref, what=f"mfma verify col {j}")
