"""Seeded input generators: determinism, published SplitMix64 outputs,
distributions and shapes (CPU only)."""
import os

import numpy as np

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
