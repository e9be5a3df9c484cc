"""Pins of the oracle's sliding-window layers (the "Muse Spark Open"
article, section on how the model is split: most layers attend over the
last 2,048 tokens, the rest globally).  Reading: a layer of window W lets
the token at position p attend [max(0, p - W + 1), p], its own included.

Each pin holds only for that exact window: a window that included one
position too many or too few fails the boundary perturbation, and W = 1
reduces attention to the token's own V (softmax over one score is 1), which
leaves the logits independent of the position and of all history."""
import numpy as np
import pytest

from oracle import OracleCache, OracleModel
from oracle.decode import window_start
from synth import gen
from synth.configs import DecodeConfig

CFG = DecodeConfig(name="win", n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                   vocab=37, prefill=12, n_decode=4, weight_sigma=0.3)


def test_window_start_cases():
    assert window_start(10, 0) == 0          # global
    assert window_start(10, 1) == 10         # only itself
    assert window_start(10, 3) == 8          # 8, 9, 10
    assert window_start(10, 11) == 0         # exactly all positions
    assert window_start(10, 12) == 0
    assert window_start(0, 5) == 0


def _cache(cfg, bump=None):
    c = OracleCache(cfg.n_layers, cfg.max_pos, cfg.n_kv_heads, cfg.head_dim)
    for li in range(cfg.n_layers):
        k, v = gen.kv_prefill_bf16(cfg, li)
        c.k[li][:cfg.prefill] = k
        c.v[li][:cfg.prefill] = v
    if bump is not None:   # flip K and V bits of one cached position in every layer
        for li in range(cfg.n_layers):
            c.k[li][bump] ^= np.uint16(0x0040)
            c.v[li][bump] ^= np.uint16(0x0040)
    return c


def _logits(cfg, T, token, pos, bump=None):
    return OracleModel(cfg, T).step(_cache(cfg, bump), token, pos)


def test_window_covering_everything_is_global():
    T = gen.dense_weights(CFG)
    pos = CFG.prefill
    ref = _logits(CFG, T, 5, pos)
    for w in ((pos + 1, pos + 1), (10 ** 6, 0), (0, pos + 1)):
        assert np.array_equal(_logits(CFG.with_(layer_window=w), T, 5, pos), ref)
    # one position short of everything is not global
    assert not np.array_equal(_logits(CFG.with_(layer_window=(pos, pos)), T, 5, pos), ref)


@pytest.mark.parametrize("w", [1, 3, 7])
def test_window_boundary_by_perturbation(w):
    cfg = CFG.with_(layer_window=(w, w))
    T = gen.dense_weights(cfg)
    pos = cfg.prefill
    ref = _logits(cfg, T, 5, pos)
    # the last position outside the window does not matter ...
    assert np.array_equal(_logits(cfg, T, 5, pos, bump=pos - w), ref)
    # ... the first one inside it does
    if w > 1:
        assert not np.array_equal(_logits(cfg, T, 5, pos, bump=pos - w + 1), ref)


def test_window_one_is_own_value_only():
    cfg = CFG.with_(layer_window=(1, 1))
    T = gen.dense_weights(cfg)
    a = _logits(cfg, T, 7, cfg.prefill)
    b = _logits(cfg, T, 7, 3, bump=1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # the global model does depend on the position
    g = CFG
    assert not np.allclose(_logits(g, T, 7, g.prefill), _logits(g, T, 7, 3), rtol=1e-6, atol=1e-6)
