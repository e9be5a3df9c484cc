"""GPU parity of the standalone LM-head GEMV + argmax and of the online FP8
row quantiser, through the C-ABI, against the CPU oracle."""
import numpy as np
import pytest

from gpu_util import check_argmax, compare_logits, say
from oracle import codecs, quantize_fp8_rows
from synth import CONFIGS, gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _M():
    from memory_bound_gemv_amd import _mbg
    return _mbg


def _dev_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _run_lm(w_tensor, x_np, V):
    M = _M()
    k = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np, dtype=np.float32)).cuda()
    logits = torch.empty((k, V), dtype=torch.float32, device="cuda")
    amax = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    nbytes = M.mbg_lm_head_workspace_size(k)
    ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    M.mbg_lm_head(w_tensor, x, k, logits, amax, ws, nbytes, s)
    torch.cuda.synchronize()
    # the workspace is left zeroed for the next call
    assert int(ws.abs().sum()) == 0
    return logits.cpu().numpy(), amax.cpu().numpy()


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_lm_head_bf16_ragged(k):
    V, H = 1037, 256     # V not a multiple of the wave count; K < 512
    say("lm_head bf16 ragged", V, H, k)
    w = gen.normal_bf16("t.lm_small", (V, H), 0.02)
    x = np.random.default_rng(k).standard_normal((k, H)).astype(np.float32)
    M = _M()
    wd = _dev_bits(w)
    got, idx = _run_lm(M.make_tensor(wd, "bf16", V, H), x, V)
    ref = x.astype(np.float64) @ codecs.bf16_to_f64(w).T
    for j in range(k):
        compare_logits(got[j], ref[j], what=f"col {j}")
        check_argmax(int(idx[j]), got[j], ref[j], what=f"col {j}")


def test_lm_head_onehot_dequant_is_exact():
    """x = e_j gives column j as one product plus zeros: exact in binary32."""
    V, H = 700, 512
    rng = np.random.default_rng(3)
    w = gen.normal_bf16("t.onehot", (V, H), 0.02)
    M = _M()
    wd = _dev_bits(w)
    cols = [0, 1, 7, 8, 255, 256, 511]
    x = np.zeros((len(cols), H), dtype=np.float32)
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    say("one-hot bf16")
    for g in range(0, len(cols), 4):
        got, _ = _run_lm(M.make_tensor(wd, "bf16", V, H), x[g:g + 4], V)
        for r, c in enumerate(cols[g:g + 4]):
            want = codecs.bf16_to_f64(w[:, c]).astype(np.float32)
            assert np.array_equal(got[r].astype(np.float32), want), f"bf16 column {c}"
    # FP8: codes from the GPU quantiser must equal the oracle's, and the
    # one-hot logits must be decode(code) * scale rounded once in binary32
    codes = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((V,), dtype=torch.float32, device="cuda")
    M.mbg_quantize_fp8_rows(wd, V, H, codes, scales, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs = quantize_fp8_rows(w)
    assert np.array_equal(codes.cpu().numpy(), rc), "fp8 codes"
    assert np.array_equal(scales.cpu().numpy(), rs), "fp8 scales"
    say("one-hot fp8")
    for g in range(0, len(cols), 4):
        got, _ = _run_lm(M.make_tensor(codes, "fp8", V, H, scale=scales), x[g:g + 4], V)
        for r, c in enumerate(cols[g:g + 4]):
            want = (codecs.fp8e4m3_to_f64(rc[:, c]).astype(np.float32) * rs).astype(np.float32)
            assert np.array_equal(got[r].astype(np.float32), want), f"fp8 column {c}"


def test_quantize_fp8_rows_edge_rows():
    """Zero rows, saturation-adjacent values, subnormal codes, ties."""
    H = 64
    rows = []
    rows.append(np.zeros(H, dtype=np.float32))
    r = np.zeros(H, dtype=np.float32); r[5] = -3.0; rows.append(r)
    rows.append(np.linspace(-1, 1, H).astype(np.float32))
    rows.append((np.arange(H) * 2.0 ** -12).astype(np.float32))
    rows.append(np.random.default_rng(0).standard_normal(H).astype(np.float32) * 1e-3)
    w = (np.stack(rows).view(np.uint32) >> 16).astype(np.uint16)
    M = _M()
    wd = _dev_bits(w)
    codes = torch.empty(w.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((w.shape[0],), dtype=torch.float32, device="cuda")
    M.mbg_quantize_fp8_rows(wd, w.shape[0], H, codes, scales, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rc, rs = quantize_fp8_rows(w)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)


@pytest.mark.parametrize("k", [1, 4])
def test_lm_head_full_size_bf16(k):
    cfg = CONFIGS["lmhead"]
    say("lm_head full bf16", cfg.vocab, cfg.hidden, k)
    w = gen.lm_head_bf16(cfg)
    x = gen.lm_head_inputs(cfg, k)
    M = _M()
    wd = _dev_bits(w)
    got, idx = _run_lm(M.make_tensor(wd, "bf16", cfg.vocab, cfg.hidden), x, cfg.vocab)
    ref = np.empty((k, cfg.vocab))
    xd = x.astype(np.float64)
    for r0 in range(0, cfg.vocab, 16384):
        ref[:, r0:r0 + 16384] = xd @ codecs.bf16_to_f64(w[r0:r0 + 16384]).T
    for j in range(k):
        compare_logits(got[j], ref[j], what=f"col {j}")
        check_argmax(int(idx[j]), got[j], ref[j], what=f"col {j}")


@pytest.mark.timeout(900)
def test_lm_head_full_size_fp8():
    """The full 157,184 x 2,560 head quantised to FP8 by the library: every
    row's codes and scale equal the oracle's quantiser, and for k = 1 and 4
    every logit matches the oracle's dequantise-then-dot, with the argmax
    graded against the oracle's wherever its top-2 margin exceeds 1e-2."""
    cfg = CONFIGS["lmhead"]
    say("lm_head full fp8")
    w = gen.lm_head_bf16(cfg)
    M = _M()
    wd = _dev_bits(w)
    V, H = cfg.vocab, cfg.hidden
    codes = torch.empty((V, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((V,), dtype=torch.float32, device="cuda")
    M.mbg_quantize_fp8_rows(wd, V, H, codes, scales, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del wd
    xs = {k: gen.lm_head_inputs(cfg, k) for k in (1, 4)}
    got = {k: _run_lm(M.make_tensor(codes, "fp8", V, H, scale=scales), xs[k], V) for k in (1, 4)}
    gc = codes.cpu().numpy()
    gs = scales.cpu().numpy()
    ref = {k: np.empty((k, V)) for k in (1, 4)}
    chunk = 16384
    for r0 in range(0, V, chunk):
        rc, rs = quantize_fp8_rows(w[r0:r0 + chunk])
        assert np.array_equal(gc[r0:r0 + chunk], rc), f"codes of rows {r0}.."
        assert np.array_equal(gs[r0:r0 + chunk], rs), f"scales of rows {r0}.."
        deq = codecs.fp8e4m3_to_f64(rc) * rs.astype(np.float64)[:, None]
        for k in (1, 4):
            ref[k][:, r0:r0 + chunk] = xs[k].astype(np.float64) @ deq.T
        say(f"rows {r0}..{min(V, r0 + chunk)} checked")
    graded = 0
    for k in (1, 4):
        g, idx = got[k]
        for j in range(k):
            compare_logits(g[j], ref[k][j], what=f"k {k} col {j}")
            graded += check_argmax(int(idx[j]), g[j], ref[k][j], what=f"k {k} col {j}")
    say("fp8 head argmax graded", graded, "of 5")
