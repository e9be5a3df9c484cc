"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-only validation rejects bad input with the right code
(no device call is made)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def M():
    from memory_bound_gemv_amd import _mbg
    return _mbg


def _declared():
    src = open(os.path.join(ROOT, "include", "mbg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mbg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_and_library_exports(M):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(M._lib, n), n
    assert sorted(M.EXPORTED) == names


def _cfg(M, **kw):
    base = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=1024, vocab=4096,
                max_pos=48, k_max=4)
    base.update(kw)
    return M.make_config(**base)


def test_validate_config_errors(M):
    assert M.mbg_validate(_cfg(M)) == 0
    assert M.mbg_validate(_cfg(M, head_dim=96)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, hidden=250)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, n_q_heads=5)) == M.MBG_E_INVALID_ARG
    assert M.mbg_validate(_cfg(M, k_max=5)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, k_max=0)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, n_layers=0)) == M.MBG_E_INVALID_ARG
    assert M.mbg_validate(_cfg(M, max_pos=0)) == M.MBG_E_INVALID_ARG
    assert M.mbg_validate(_cfg(M, ffn=0)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, n_experts=8, top_k=9, moe_ffn=64)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, n_experts=8, top_k=2, moe_ffn=48)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, layer_window=[0, 2048])) == 0
    assert M.mbg_validate(_cfg(M, layer_window=[1, 0])) == 0
    assert M.mbg_validate(_cfg(M, layer_window=[5, -1])) == M.MBG_E_INVALID_ARG
    # KV pages: a power of two of at least 16 positions (an attention
    # instruction reads up to 16 consecutive positions from one page)
    for ps in (16, 32, 64, 256):
        assert M.mbg_validate(_cfg(M, page_size=ps)) == 0, ps
    for ps in (8, 12, 48, 96):
        assert M.mbg_validate(_cfg(M, page_size=ps)) == M.MBG_E_UNSUPPORTED, ps
    assert M.mbg_validate(_cfg(M, page_size=0)) == M.MBG_E_INVALID_ARG
    M.mbg_validate(_cfg(M, page_size=48))
    assert "page_size 48" in M.mbg_last_error()
    M.mbg_validate(_cfg(M, head_dim=96))
    assert "head_dim 96" in M.mbg_last_error()


FAKE = 0x10000   # a 16-byte-aligned address; validation never dereferences it


def _weights(M, cfg_kw=None, lm_dtype="bf16", mutate=None):
    c = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=1024, vocab=4096)
    H, d = 256, 64
    T = M.make_tensor
    layers = []
    for _ in range(2):
        lay = dict(attn_norm=T(FAKE, "bf16", 1, H), ffn_norm=T(FAKE, "bf16", 1, H),
                   wq=T(FAKE, "bf16", 4 * d, H), wk=T(FAKE, "bf16", 2 * d, H), wv=T(FAKE, "bf16", 2 * d, H),
                   wo=T(FAKE, "bf16", H, 4 * d), w_gate=T(FAKE, "bf16", 1024, H), w_up=T(FAKE, "bf16", 1024, H),
                   w_down=T(FAKE, "bf16", H, 1024))
        if mutate:
            mutate(lay)
        layers.append(M.make_layer(**lay))
    lm = T(FAKE, "fp8", 4096, H, scale=FAKE) if lm_dtype == "fp8" else T(FAKE, "bf16", 4096, H)
    return M.WeightSet(layers, T(FAKE, "bf16", 4096, H), T(FAKE, "bf16", 1, H), lm)


def test_validate_weights(M):
    cfg = _cfg(M)
    assert M.mbg_validate(cfg, _weights(M)) == 0
    assert M.mbg_validate(cfg, _weights(M, lm_dtype="fp8")) == 0

    def wrong_dtype(l):
        l["wq"] = M.make_tensor(FAKE, "fp8", 256, 256, scale=FAKE)
    assert M.mbg_validate(cfg, _weights(M, mutate=wrong_dtype)) == M.MBG_E_DTYPE_MISMATCH

    def wrong_shape(l):
        l["wo"] = M.make_tensor(FAKE, "bf16", 256, 255)
    assert M.mbg_validate(cfg, _weights(M, mutate=wrong_shape)) == M.MBG_E_INVALID_ARG

    def null(l):
        l["w_down"] = M.make_tensor(None, "bf16", 256, 1024)
    assert M.mbg_validate(cfg, _weights(M, mutate=null)) == M.MBG_E_INVALID_ARG

    def misaligned(l):
        l["w_up"] = M.make_tensor(FAKE + 2, "bf16", 1024, 256)
    assert M.mbg_validate(cfg, _weights(M, mutate=misaligned)) == M.MBG_E_INVALID_ARG

    def bf16_with_scale(l):
        l["wk"] = M.make_tensor(FAKE, "bf16", 128, 256, scale=FAKE)
    assert M.mbg_validate(cfg, _weights(M, mutate=bf16_with_scale)) == M.MBG_E_DTYPE_MISMATCH

    # an FP8 LM head without its scale is the silent-fallback case: rejected
    w = _weights(M)
    w.struct.lm_head = M.make_tensor(FAKE, "fp8", 4096, 256)
    assert M.mbg_validate(cfg, w) == M.MBG_E_DTYPE_MISMATCH


def test_validate_kv(M):
    cfg = _cfg(M)
    ok = M.make_kv("bf16", 1, FAKE, FAKE)
    assert M.mbg_validate(cfg, None, ok) == 0
    # FP8 KV is compiled for the 2B dense shape
    cfg128 = _cfg(M, hidden=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=8192, vocab=32000)
    assert M.mbg_validate(cfg128, None, M.make_kv("fp8", 1, FAKE, FAKE)) == M.MBG_E_DTYPE_MISMATCH
    assert M.mbg_validate(cfg128, None, M.make_kv("fp8", 1, FAKE, FAKE, FAKE)) == 0
    assert M.mbg_validate(cfg, None, M.make_kv("bf16", 1, FAKE, FAKE, FAKE)) == M.MBG_E_DTYPE_MISMATCH
    assert M.mbg_validate(cfg, None, M.make_kv("mxfp4", 1, FAKE, FAKE)) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(cfg, None, M.make_kv("bf16", 0, FAKE, FAKE)) == M.MBG_E_INVALID_ARG
    assert M.mbg_validate(cfg, None, M.make_kv("bf16", 1, None, FAKE)) == M.MBG_E_INVALID_ARG
    # no compiled kernel for 3 query heads per KV head, nor for other widths
    assert M.mbg_validate(_cfg(M, n_q_heads=6), None, ok) == M.MBG_E_UNSUPPORTED
    assert M.mbg_validate(_cfg(M, ffn=2048), None, ok) == M.MBG_E_UNSUPPORTED
    assert "no compiled kernel" in M.mbg_last_error()


def test_workspace_size_grows_with_window(M):
    a = M.mbg_workspace_size(_cfg(M, k_max=1))
    b = M.mbg_workspace_size(_cfg(M, k_max=4))
    assert 0 < a < b
    with pytest.raises(M.MbgError) as e:
        M.mbg_workspace_size(_cfg(M, head_dim=32))
    assert e.value.code == M.MBG_E_UNSUPPORTED


def test_standalone_argument_errors(M):
    with pytest.raises(M.MbgError) as e:
        M.mbg_lm_head_workspace_size(5)
    assert e.value.code == M.MBG_E_RANGE
    for w in (M.make_tensor(FAKE, "fp32", 100, 256),                 # no fp32 rows
              M.make_tensor(FAKE, "mxfp4", 100, 48, scale=FAKE)):    # MXFP4 blocks are 32 wide
        with pytest.raises(M.MbgError) as e:
            M.mbg_lm_head(w, FAKE, 1, FAKE, FAKE, FAKE, 256, 0)
        assert e.value.code == M.MBG_E_UNSUPPORTED
    with pytest.raises(M.MbgError) as e:
        M.mbg_quantize_fp8_rows(FAKE, 10, 20, FAKE, FAKE, 0)
    assert e.value.code == M.MBG_E_INVALID_ARG


def _kv_ok(M):
    return M.make_kv("bf16", 1, FAKE, FAKE)


def test_counter_block_size_and_init_ownership_checks(M):
    """The caller owns the counter block: init rejects a missing, short or
    misaligned one before touching the device (host-side checks only)."""
    cfg = _cfg(M)
    n = M.mbg_counter_bytes(cfg)
    L = 2
    assert n == 128 + (L * 6 + 1) * 8 * 128   # status line + 8 lines per (layer, phase) counter + step token
    assert M.mbg_counter_bytes(_cfg(M, n_layers=64)) < 1 << 20
    ws = M.mbg_workspace_size(cfg)
    for ctr, nbytes in ((None, n), (FAKE, n - 4), (FAKE + 16, n)):
        with pytest.raises(M.MbgError) as e:
            M.mbg_decode_init(cfg, _weights(M), _kv_ok(M), FAKE, ws, ctr, nbytes, 0)
        assert e.value.code == M.MBG_E_WORKSPACE, M.mbg_last_error()
        assert "counter block" in M.mbg_last_error()
    with pytest.raises(M.MbgError) as e:
        M.mbg_decode_init(cfg, _weights(M), _kv_ok(M), FAKE, ws - 256, FAKE, n, 0)
    assert e.value.code == M.MBG_E_WORKSPACE and "workspace" in M.mbg_last_error()


def test_header_states_ownership_and_passages():
    """Every declared entry point's comment cites a page passage (or, for the
    no-allocation variant, names the callers it is for), and the header says
    that no call allocates device memory."""
    src = open(os.path.join(ROOT, "include", "mbg.h")).read()
    assert "No call allocates or frees device" in src
    assert "never allocates" not in src
    blocks = re.findall(r"/\*((?:(?!\*/).)*?)\*/\s*(?:const char \*|void|int)\s*\*?\s*(mbg_[a-z0-9_]+)\s*\(",
                        src, flags=re.S)
    seen = {name for _, name in blocks}
    assert set(_declared()) <= seen
    for text, name in blocks:
        cites = any(w in text for w in ("article", "report", "cannot allocate"))
        if name in ("mbg_last_error", "mbg_query", "mbg_read_trace", "mbg_read_routing",
                    "mbg_lm_head_workspace_size"):
            continue    # accessors of what another call documented
        assert cites, f"{name}: no passage cited"
