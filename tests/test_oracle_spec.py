"""Pins of the oracle's speculative round (163.com Ling-3.0-flash article,
optimisation 3: draft, one-pass verify of the window, greedy acceptance of
the agreeing prefix).

Greedy acceptance makes the emitted tokens those of greedy decoding of the
target, whatever the draft proposes: only the number of tokens per round
depends on the draft.  So the rounds are pinned against plain greedy steps
of the target (for an early-exit draft and for a draft that is always
wrong), a draft that is the target itself has every token accepted, and an
always-wrong draft has none accepted."""
import numpy as np
import pytest

from oracle import OracleCache, OracleModel
from oracle.decode import argmax_lower_index, spec_round
from synth import gen
from synth.configs import DecodeConfig

CFG = DecodeConfig(name="spec", n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                   vocab=37, prefill=6, n_decode=40, weight_sigma=0.3)


def _models():
    T = gen.dense_weights(CFG)
    target = OracleModel(CFG, T)
    dcfg = CFG.with_(n_layers=1)
    early = OracleModel(dcfg, {k: v for k, v in T.items() if not k.startswith("l1.")})
    return T, target, dcfg, early


def _cache(cfg):
    c = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    for li in range(cfg.n_layers):
        k, v = gen.kv_prefill_bf16(CFG, li)
        c.k[li][:CFG.prefill] = k
        c.v[li][:CFG.prefill] = v
    return c


def _greedy(target, n, token, pos):
    c = _cache(CFG)
    out = []
    for i in range(n):
        token = argmax_lower_index(target.step(c, token, pos + i))
        out.append(token)
    return out


class _Wrong:
    """A draft that always proposes the token after the target's greedy one
    (so it is never accepted); it reads the target's logits to know it."""

    def __init__(self, target, cfg):
        self.target, self.cache = target, _cache(cfg)

    def step(self, _cache_unused, token, pos):
        lg = self.target.step(self.cache, token, pos)
        z = np.full(CFG.vocab, -1.0)
        z[(argmax_lower_index(lg) + 1) % CFG.vocab] = 1.0
        return z


def _rounds(target, draft, dcache, k, n_tokens):
    tc = _cache(CFG)
    tok, pos = 5, CFG.prefill
    out, ms = [], []
    while len(out) < n_tokens:
        em, pos, tok, win, _ = spec_round(target, tc, draft, dcache, tok, pos, k)
        out += em
        ms.append(len(em) - 1)
    return out[:n_tokens], ms


@pytest.mark.parametrize("k", [2, 4])
def test_early_exit_draft_emits_greedy_tokens(k):
    _, target, dcfg, early = _models()
    out, ms = _rounds(target, early, _cache(dcfg), k, 24)
    assert out == _greedy(target, 24, 5, CFG.prefill)
    assert all(0 <= m <= k - 1 for m in ms)


def test_target_as_draft_accepts_everything():
    _, target, _, _ = _models()
    out, ms = _rounds(target, target, _cache(CFG), 4, 24)
    assert out == _greedy(target, 24, 5, CFG.prefill)
    assert all(m == 3 for m in ms)


def test_wrong_draft_accepts_nothing():
    _, target, _, _ = _models()
    wrong = _Wrong(target, CFG)
    out, ms = _rounds(target, wrong, None, 4, 12)
    assert out == _greedy(target, 12, 5, CFG.prefill)
    assert all(m == 0 for m in ms)
