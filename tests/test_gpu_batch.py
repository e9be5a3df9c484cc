"""GPU parity of batches of independent sequences (mbg_decode_batch; the
"Muse Spark Open" article, section on what would change the result, names
batch > 1 first).  Sequences share the pool on disjoint pages; column i of
a batch decodes sequence seq[i] at pos[i] and must equal that sequence's own
oracle step: nothing of another sequence's cache or tokens may reach it."""
import numpy as np
import pytest

from gpu_util import LOGIT_REL_L2_MXFP4, build_dense, build_moe, check_argmax, compare_logits, say
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _batch_steps(dm, om, ocs, cfg, seqs, pos0, first, n_steps, what, rel_tol=None):
    """n_steps batch calls over sequences `seqs` starting at positions pos0;
    column i starts with token first[i] and continues with its own argmax.
    Each column is compared with the oracle step of its sequence."""
    n = len(seqs)
    toks = torch.tensor(first, dtype=torch.int32, device="cuda")
    logits = torch.empty((n, cfg.vocab), dtype=torch.float32, device="cuda")
    am = torch.zeros(n, dtype=torch.int32, device="cuda")
    kw = {} if rel_tol is None else {"rel_tol": rel_tol}
    cur = [int(t) for t in first]
    pos = list(pos0)
    graded = 0
    for s in range(n_steps):
        toks.copy_(torch.tensor(cur, dtype=torch.int32))
        dm.batch(toks, seqs, pos, logits, am)
        torch.cuda.synchronize()
        g, amh = logits.cpu().numpy(), am.cpu().numpy()
        for i, b in enumerate(seqs):
            ref = om.step(ocs[b], cur[i], pos[i])
            compare_logits(g[i], ref, what=f"{what} step {s} col {i} seq {b} pos {pos[i]}", **kw)
            graded += check_argmax(int(amh[i]), g[i], ref, what=f"{what} step {s} col {i}")
        cur = [int(a) for a in amh]
        pos = [p + 1 for p in pos]
    assert dm.status() == 0
    return pos, cur, graded


def test_tiny_batch_sequences():
    cfg = CONFIGS["tiny"].with_(prefill=24, n_prompt=0, n_decode=24, layer_window=(0, 9))
    lens = [24, 5, 17, 0]
    say("tiny batch", lens)
    dm, om, ocs = build_dense(cfg, prefill_lens=lens)
    prompt = gen.prompt_tokens(cfg, 8)
    # one-column batches extend sequence 3 alone (a sequence other than 0)
    pos, cur, _ = _batch_steps(dm, om, ocs, cfg, [3], [0], [int(prompt[0])], 4, "tiny seq3")
    # all four sequences together, each at its own position
    p4 = [lens[0], lens[1], lens[2], pos[0]]
    first = [int(t) for t in prompt[1:5]]
    p4, cur4, graded = _batch_steps(dm, om, ocs, cfg, [0, 1, 2, 3], p4, first, 5, "tiny batch4")
    assert graded >= 12
    # permuted and partial mappings continue the same sequences
    p2, _, _ = _batch_steps(dm, om, ocs, cfg, [2, 0], [p4[2], p4[0]], [cur4[2], cur4[0]], 2, "tiny batch [2,0]")
    _batch_steps(dm, om, ocs, cfg, [3, 1, 2], [p4[3], p4[1], p2[0]], [cur4[3], cur4[1], 7], 2, "tiny batch [3,1,2]")


def test_batch_argument_checks():
    cfg = CONFIGS["tiny"].with_(prefill=8, n_prompt=0, n_decode=8)
    dm, _, _ = build_dense(cfg, prefill_lens=[8, 8])
    toks = torch.zeros(2, dtype=torch.int32, device="cuda")
    am = torch.zeros(2, dtype=torch.int32, device="cuda")
    from memory_bound_gemv_amd import _mbg as M
    for seq, pos in (([0, 0], [8, 8]), ([0, 2], [8, 8]), ([0, 1], [8, cfg.max_pos]), ([0, -1], [8, 8])):
        with pytest.raises(Exception):
            dm.batch(toks, seq, pos, None, am)
    with pytest.raises(Exception):   # more columns than the context's widest window
        M.mbg_decode_batch(dm.ctx, toks, 5, [0, 1, 0, 1, 0], [1, 1, 1, 1, 1], None, am)
    dm.batch(toks, [1, 0], [8, 8], None, am)
    torch.cuda.synchronize()
    assert dm.status() == 0


def test_dense2b_batch4():
    cfg = CONFIGS["dense2b"]
    lens = [4096, 3001, 2048, 999]
    say("dense2b batch build", lens)
    dm, om, ocs = build_dense(cfg, prefill_lens=lens)
    first = [int(t) for t in gen.prompt_tokens(cfg, 4)]
    _, _, graded = _batch_steps(dm, om, ocs, cfg, [0, 1, 2, 3], lens, first, 3, "dense2b batch4")
    say("dense2b batch graded", graded)
    assert graded >= 8


def test_dense2b_fp8_kv_batch4():
    """FP8 caches (the long-context kernel family) on shuffled pages, with
    sliding-window layers."""
    base = CONFIGS["dense2b"].with_(kv_dtype="fp8", prefill=2048, n_decode=8, shuffled_pages=True)
    cfg = base.with_(layer_window=tuple(0 if li % 4 == 3 else 700 for li in range(base.n_layers)))
    lens = [2048, 700, 1500, 33]
    say("dense2b fp8 batch build", lens)
    dm, om, ocs = build_dense(cfg, prefill_lens=lens)
    first = [int(t) for t in gen.prompt_tokens(cfg, 4)]
    _, _, graded = _batch_steps(dm, om, ocs, cfg, [1, 3, 0, 2], [lens[1], lens[3], lens[0], lens[2]], first, 2,
                                "dense2b fp8 batch4")
    say("dense2b fp8 batch graded", graded)


def test_moe_small_batch4():
    cfg = CONFIGS["moe"].with_(name="moe_small", n_layers=2, n_experts=64, vocab=4096, prefill=256, n_decode=8)
    lens = [256, 100, 200, 17]
    say("moe_small batch build", lens)
    dm, om, ocs = build_moe(cfg, prefill_lens=lens)
    first = [int(t) for t in gen.prompt_tokens(cfg, 4)]
    _batch_steps(dm, om, ocs, cfg, [3, 1, 0, 2], [lens[3], lens[1], lens[0], lens[2]], first, 3, "moe_small batch4",
                 rel_tol=LOGIT_REL_L2_MXFP4)
