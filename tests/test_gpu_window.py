"""GPU parity of sliding-window attention layers (the "Muse Spark Open"
article, section on how the model is split: layers attending over the last
2,048 tokens next to global ones) against the oracle, whose window bound the
CPU tests pin.  A layer of window W lets position p attend
[max(0, p - W + 1), p]."""
import numpy as np
import pytest

from gpu_util import LOGIT_REL_L2_MXFP4, build_dense, build_moe, check_argmax, compare_logits, say
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")



def _steps(dm, om, oc, cfg, p0, tokens, n, greedy_from, what, rel_tol=None):
    """n teacher-forced steps from p0: tokens[i] for i < greedy_from, then
    the GPU's argmax.  Returns the number of graded argmax decisions."""
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    nxt, graded = int(tokens[0]), 0
    kw = {} if rel_tol is None else {"rel_tol": rel_tol}
    for i in range(n):
        t = int(tokens[i]) if i < greedy_from else nxt
        tok.fill_(t)
        dm.step(tok, p0 + i, logits, amax)
        torch.cuda.synchronize()
        g = logits.cpu().numpy()
        ref = om.step(oc, t, p0 + i)
        compare_logits(g, ref, what=f"{what} step {i} pos {p0 + i}", **kw)
        graded += check_argmax(int(amax.item()), g, ref, what=f"{what} step {i}")
        nxt = int(amax.item())
    assert dm.status() == 0
    return graded


@pytest.mark.parametrize("windows", [(5, 0), (1, 17), (64, 3)])
def test_tiny_window_sequence(windows):
    cfg = CONFIGS["tiny"].with_(layer_window=windows)
    say("tiny window", windows)
    dm, om, oc = build_dense(cfg)
    prompt = gen.prompt_tokens(cfg, cfg.n_prompt)
    graded = _steps(dm, om, oc, cfg, 0, prompt, cfg.n_prompt + cfg.n_decode, cfg.n_prompt, f"tiny w{windows}")
    assert graded >= 40


@pytest.mark.parametrize("k", [2, 4])
def test_tiny_window_verify(k):
    """A window narrower than the verify window: column j must not see the
    window's tokens more than W - 1 positions back."""
    cfg = CONFIGS["tiny"].with_(layer_window=(2, 3))
    say("tiny window verify", k)
    dm, om, oc = build_dense(cfg)
    prompt = gen.prompt_tokens(cfg, 40)
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    amax = torch.zeros(1, dtype=torch.int32, device="cuda")
    p0 = 20
    for pos in range(p0):
        tok.fill_(int(prompt[pos]))
        dm.step(tok, pos, None, amax)
        om.step(oc, int(prompt[pos]), pos)
    win = torch.from_numpy(prompt[p0:p0 + k].astype(np.int32)).cuda()
    logits = torch.empty((k, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(k, dtype=torch.int32, device="cuda")
    dm.verify(win, p0, logits, am)
    torch.cuda.synchronize()
    ref = om.verify(oc, [int(t) for t in prompt[p0:p0 + k]], p0)
    g, amh = logits.cpu().numpy(), am.cpu().numpy()
    for j in range(k):
        compare_logits(g[j], ref[j], what=f"window verify col {j}")
        check_argmax(int(amh[j]), g[j], ref[j], what=f"window verify col {j}")
    assert dm.status() == 0


def test_window_covering_everything_is_global_bitwise():
    """Windows wider than every position take the global kernel path's exact
    arithmetic (same splits, nothing masked)."""
    base = CONFIGS["tiny"]
    say("tiny wide window vs global")
    outs = []
    for cfg in (base, base.with_(layer_window=(10 ** 6, 10 ** 6))):
        dm, _, _ = build_dense(cfg)
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        lg = torch.empty(cfg.vocab, dtype=torch.float32, device="cuda")
        am = torch.zeros(1, dtype=torch.int32, device="cuda")
        seq = []
        for pos, t in enumerate(gen.prompt_tokens(cfg, 24)):
            tok.fill_(int(t))
            dm.step(tok, pos, lg, am)
            seq.append(lg.cpu().numpy().copy())
        assert dm.status() == 0
        outs.append(np.stack(seq))
    assert np.array_equal(outs[0], outs[1])


def test_dense2b_window_steps():
    """The dense 2B workload at 4096 with windows of 512 on even layers, 1 on
    layer 3 and global elsewhere."""
    base = CONFIGS["dense2b"]
    win = tuple(512 if li % 2 == 0 else (1 if li == 3 else 0) for li in range(base.n_layers))
    cfg = base.with_(layer_window=win)
    say("dense2b window build")
    dm, om, oc = build_dense(cfg)
    toks = gen.prompt_tokens(cfg, 4)
    graded = _steps(dm, om, oc, cfg, cfg.prefill, toks, 4, 2, "dense2b window")
    say("dense2b window graded", graded)


def test_longctx_window_steps():
    """FP8 cache at 200,000 on shuffled pages: three of every four layers
    attend over the last 2,048 positions, the fourth globally; two steps
    (the second reads the K/V the first wrote)."""
    base = CONFIGS["longctx"]
    win = tuple(0 if li % 4 == 3 else 2048 for li in range(base.n_layers))
    cfg = base.with_(layer_window=win)
    say("longctx window build")
    dm, om, oc = build_dense(cfg)
    toks = gen.prompt_tokens(cfg, 1)
    _steps(dm, om, oc, cfg, cfg.prefill, toks, 2, 1, "longctx window")


def test_moe_small_window_steps_and_verify():
    base = CONFIGS["moe"].with_(name="moe_small", n_layers=2, n_experts=64, vocab=4096, prefill=256, n_decode=8)
    cfg = base.with_(layer_window=(100, 0))
    say("moe_small window build")
    dm, om, oc = build_moe(cfg)
    toks = gen.prompt_tokens(cfg, 4)
    steps = []
    _steps(dm, om, oc, cfg, cfg.prefill, toks, 4, 4, "moe_small window", rel_tol=LOGIT_REL_L2_MXFP4)
    # the same four tokens as one verify window on a fresh model
    dm2, om2, oc2 = build_moe(cfg)
    ref = om2.verify(oc2, [int(t) for t in toks], cfg.prefill)
    win = torch.from_numpy(np.asarray(toks, dtype=np.int32)).cuda()
    logits = torch.empty((4, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(4, dtype=torch.int32, device="cuda")
    dm2.verify(win, cfg.prefill, logits, am)
    torch.cuda.synchronize()
    g = logits.cpu().numpy()
    for j in range(4):
        compare_logits(g[j], ref[j], rel_tol=LOGIT_REL_L2_MXFP4, what=f"moe_small window verify col {j}")
    assert dm2.status() == 0
