"""Seeded input generators: determinism, published SplitMix64 outputs,
distributions and shapes (CPU only)."""
import os

import numpy as np
import pytest

from synth import CONFIGS, gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_outputs():
    want = []
    with open(os.path.join(GOLDEN, "splitmix64_seed0.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                want.append(int(line, 16))
    with np.errstate(over="ignore"):
        states = np.arange(1, 4, dtype=np.uint64) * gen.GOLDEN_GAMMA
    got = [int(v) for v in gen.splitmix64(states)]
    assert got == want


def test_weights_are_deterministic_and_distinct():
    a = gen.normal_bf16("x.w", (64, 64), 0.02)
    b = gen.normal_bf16("x.w", (64, 64), 0.02)
    c = gen.normal_bf16("x.v", (64, 64), 0.02)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    v = (a.astype(np.uint32) << 16).view(np.float32)
    assert abs(v.std() - 0.02) < 0.002 and abs(v.mean()) < 0.002


def test_page_table_is_a_permutation():
    cfg = CONFIGS["longctx"]
    pt = gen.page_table(cfg)
    assert pt.size == cfg.n_pages == 3126
    assert np.array_equal(np.sort(pt), np.arange(cfg.n_pages))
    assert not np.array_equal(pt, np.arange(cfg.n_pages))
    assert np.array_equal(gen.page_table(cfg, shuffled=False), np.arange(cfg.n_pages))


def test_expert_codes_uniform_and_scales_in_range():
    cfg = CONFIGS["moe"]
    codes, scales = gen.expert_mxfp4(cfg, 3, 17, "gate_up")
    assert codes.shape == (1536, 1280) and scales.shape == (1536, 80)
    nib = np.concatenate([codes & 0xF, codes >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.95 * nib.size / 16 and counts.max() < 1.05 * nib.size / 16
    assert set(np.unique(scales)) == {120, 121, 122}
    c2, s2 = gen.expert_mxfp4(cfg, 3, 17, "gate_up")
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    d, ds = gen.expert_mxfp4(cfg, 3, 17, "down")
    assert d.shape == (2560, 384) and ds.shape == (2560, 24)
    other, _ = gen.expert_mxfp4(cfg, 3, 18, "gate_up")
    assert not np.array_equal(codes, other)


def test_config_sizes():
    c = CONFIGS["dense2b"]
    assert c.max_pos == 4352 and c.qkv_rows == 4096
    assert CONFIGS["tiny"].max_pos == 48
    assert CONFIGS["longctx"].max_pos == 200064


def test_expert_hash_torch_matches_numpy():
    """The torch form of the expert generator draws the same bytes."""
    torch = pytest.importorskip("torch")
    cfg = CONFIGS["moe"].with_(hidden=256, moe_ffn=64, n_experts=16)
    for layer, e, which in ((0, 0, "gate_up"), (3, 15, "down"), (41, 16, "gate_up"), (7, 16, "down")):
        c, s = gen.expert_mxfp4(cfg, layer, e, which)
        ct = torch.empty(c.shape, dtype=torch.uint8)
        st = torch.empty(s.shape, dtype=torch.uint8)
        gen.expert_mxfp4_torch(cfg, layer, e, which, ct, st)
        assert np.array_equal(ct.numpy(), c) and np.array_equal(st.numpy(), s)
    # stacked form, several experts at once (shared expert id included)
    ids = [2, 5, 16]
    ct = torch.empty((3, 2 * cfg.moe_ffn, cfg.hidden // 2), dtype=torch.uint8)
    st = torch.empty((3, 2 * cfg.moe_ffn, cfg.hidden // 32), dtype=torch.uint8)
    gen.experts_mxfp4_torch(cfg, 9, ids, "gate_up", ct, st, chunk=2)
    for i, e in enumerate(ids):
        c, s = gen.expert_mxfp4(cfg, 9, e, "gate_up")
        assert np.array_equal(ct[i].numpy(), c) and np.array_equal(st[i].numpy(), s)
    # large stream ids and counters (the full model's last expert of its last layer)
    big = gen.hash_stream(10**6, np.arange(2**20, 2**20 + 1000, dtype=np.uint64))
    bt = gen.hash_stream_torch(10**6, 2**20, 1000, "cpu").numpy().view(np.uint64)
    assert np.array_equal(big, bt)
