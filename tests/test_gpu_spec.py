"""GPU parity of speculative rounds (mbg_spec_round; 163.com Ling-3.0-flash
article, optimisation 3): a draft context proposes k tokens, the target
verifies the window and accepts on the device, and rounds chain through a
device-resident state with no host round trip.  Each round is checked with
the GPU's own tokens fed to the oracle: the draft's tokens, the target's
window logits, and the acceptance arithmetic on the GPU's values."""
import numpy as np
import pytest

from gpu_util import (ARGMAX_MARGIN, LOGIT_REL_L2_MXFP4, build_dense, build_draft, build_moe, compare_logits,
                      lowest_argmax, say, top2_margin)
from oracle.decode import argmax_lower_index
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run_rounds(tdm, ddm, cfg, k, rounds, token, pos):
    states = torch.zeros((rounds + 1, 12), dtype=torch.int32, device="cuda")
    states[0, 0] = pos
    states[0, 4] = token
    emit = torch.zeros(rounds * k + 8, dtype=torch.int32, device="cuda")
    logits = torch.empty((rounds, k, cfg.vocab), dtype=torch.float32, device="cuda")
    for r in range(rounds):   # all enqueued; nothing read back in between
        tdm.spec_round(ddm, k, states[r], states[r + 1], emit, logits[r])
    torch.cuda.synchronize()
    assert tdm.status() == 0 and ddm.status() == 0
    return states.cpu().numpy(), emit.cpu().numpy(), logits.cpu().numpy()


def _check_rounds(cfg, k, st, emit, lg, om, oc, dom, doc, what, rel_tol=None):
    kw = {} if rel_tol is None else {"rel_tol": rel_tol}
    ms, graded = [], 0
    for r in range(len(lg)):
        cur, nxt = st[r], st[r + 1]
        pos, win = int(cur[0]), [int(t) for t in cur[4:4 + k + 1]]
        # the draft: k greedy steps from win[0]; GPU tokens fed back
        for s in range(k):
            ref = dom.step(doc, win[s], pos + s)
            if top2_margin(ref) > ARGMAX_MARGIN:
                assert win[s + 1] == argmax_lower_index(ref), f"{what} round {r} draft step {s}"
                graded += 1
        # the target's window
        ref = om.verify(oc, win[:k], pos)
        for j in range(k):
            compare_logits(lg[r][j], ref[j], what=f"{what} round {r} col {j}", **kw)
        am = [lowest_argmax(lg[r][j]) for j in range(k)]
        # acceptance, exactly, on the GPU's own values
        m = 0
        while m < k - 1 and am[m] == win[m + 1]:
            m += 1
        n0, n1 = int(cur[1]), int(nxt[1])
        assert n1 - n0 == m + 1, f"{what} round {r}: emitted {n1 - n0}, expected {m + 1}"
        assert list(emit[n0:n1]) == am[:m + 1], f"{what} round {r}: emitted {emit[n0:n1]} vs {am[:m + 1]}"
        assert int(nxt[0]) == pos + m + 1 and int(nxt[4]) == am[m]
        assert int(nxt[2]) == int(cur[2]) + m and int(nxt[3]) == int(cur[3]) + 1
        ms.append(m)
    return ms, graded


@pytest.mark.parametrize("k", [2, 4])
def test_tiny_spec_rounds_early_exit_draft(k):
    cfg = CONFIGS["tiny"].with_(prefill=24, n_prompt=0, n_decode=40)
    say("tiny spec", k)
    host = gen.dense_weights(cfg)
    tdm, om, oc = build_dense(cfg, host=host)
    ddm, dom, doc = build_draft(cfg, host, 1)
    rounds = 8
    st, emit, lg = _run_rounds(tdm, ddm, cfg, k, rounds, int(gen.prompt_tokens(cfg, 1)[0]), cfg.prefill)
    ms, graded = _check_rounds(cfg, k, st, emit, lg, om, oc, dom, doc, f"tiny spec k={k}")
    say(f"tiny spec k={k}: accepted per round {ms}, graded draft tokens {graded}")
    assert int(st[-1][3]) == rounds


def test_tiny_spec_target_as_draft_accepts():
    """The draft is the target itself: its proposals are the target's greedy
    tokens, so (up to near-ties between the one-column and the window
    arithmetic) every draft token is accepted."""
    cfg = CONFIGS["tiny"].with_(prefill=24, n_prompt=0, n_decode=40)
    host = gen.dense_weights(cfg)
    tdm, om, oc = build_dense(cfg, host=host)
    ddm, dom, doc = build_draft(cfg, host, cfg.n_layers)
    st, emit, lg = _run_rounds(tdm, ddm, cfg, 4, 6, int(gen.prompt_tokens(cfg, 1)[0]), cfg.prefill)
    ms, _ = _check_rounds(cfg, 4, st, emit, lg, om, oc, dom, doc, "tiny self-draft")
    say("tiny self-draft accepted per round", ms)
    assert sum(m == 3 for m in ms) >= 5


def test_spec_position_out_of_range_then_recovery():
    cfg = CONFIGS["tiny"].with_(prefill=24, n_prompt=0, n_decode=40)
    host = gen.dense_weights(cfg)
    tdm, _, _ = build_dense(cfg, host=host)
    ddm, _, _ = build_draft(cfg, host, 1)
    states = torch.zeros((2, 12), dtype=torch.int32, device="cuda")
    states[0, 0] = cfg.max_pos - 2   # the 4-token window would run past max_pos
    emit = torch.zeros(8, dtype=torch.int32, device="cuda")
    tdm.spec_round(ddm, 4, states[0], states[1], emit)
    torch.cuda.synchronize()
    from memory_bound_gemv_amd import _mbg as M
    assert M.mbg_get_status(ddm.ctx) == M.MBG_E_RANGE
    assert M.mbg_get_status(tdm.ctx) == M.MBG_E_RANGE
    # both contexts run normally afterwards
    states[0, 0] = cfg.prefill
    tdm.spec_round(ddm, 4, states[0], states[1], emit)
    torch.cuda.synchronize()
    assert tdm.status() == 0 and ddm.status() == 0
    assert int(states[1, 3].item()) == 1


def test_dense2b_spec_rounds():
    cfg = CONFIGS["dense2b"]
    host = gen.dense_weights(cfg)
    say("dense2b spec build")
    tdm, om, oc = build_dense(cfg, host=host)
    ddm, dom, doc = build_draft(cfg, host, 1)
    st, emit, lg = _run_rounds(tdm, ddm, cfg, 4, 4, int(gen.prompt_tokens(cfg, 1)[0]), cfg.prefill)
    ms, graded = _check_rounds(cfg, 4, st, emit, lg, om, oc, dom, doc, "dense2b spec")
    say("dense2b spec accepted per round", ms, "graded draft tokens", graded)


def test_moe_small_spec_rounds():
    cfg = CONFIGS["moe"].with_(name="moe_small", n_layers=2, n_experts=64, vocab=4096, prefill=256, n_decode=24)
    host = gen.dense_weights(cfg)
    say("moe_small spec build")
    tdm, om, oc = build_moe(cfg, host=host)
    ddm, dom, doc = build_draft(cfg, host, 1, target_dm=tdm)
    st, emit, lg = _run_rounds(tdm, ddm, cfg, 4, 3, int(gen.prompt_tokens(cfg, 1)[0]), cfg.prefill)
    ms, graded = _check_rounds(cfg, 4, st, emit, lg, om, oc, dom, doc, "moe_small spec", rel_tol=LOGIT_REL_L2_MXFP4)
    say("moe_small spec accepted per round", ms, "graded draft tokens", graded)
