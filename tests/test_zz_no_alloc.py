"""GPU test of mbg_lm_head_noalloc, the LM-head entry point for callers that
cannot allocate device memory: through the C-ABI, its output must equal
mbg_lm_head's (same kernel, workspace replaced by the library's fixed
device array) bit for bit, on two calls in a row, the second smaller; the
second call also checks that the first left the array zeroed."""
import numpy as np
import pytest

from gpu_util import check_argmax, compare_logits, say
from oracle import codecs
from synth import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _M():
    from memory_bound_gemv_amd import _mbg
    return _mbg


def _case(V, H, k, seed):
    w = gen.normal_bf16(f"t.noalloc{seed}", (V, H), 0.02)
    x = np.random.default_rng(seed).standard_normal((k, H)).astype(np.float32)
    return w, x


def test_lm_head_noalloc_matches_workspace_entry_point():
    M = _M()
    s = torch.cuda.current_stream().cuda_stream
    # second call smaller: fewer rows, fewer columns, another hidden size
    for V, H, k, seed in ((9000, 2560, 4, 1), (1037, 256, 2, 2), (3001, 2048, 1, 3)):
        say("noalloc case", V, H, k)
        w, x = _case(V, H, k, seed)
        wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).cuda()
        xd = torch.from_numpy(x).cuda()
        t = M.make_tensor(wd, "bf16", V, H)
        l_ws = torch.empty((k, V), dtype=torch.float32, device="cuda")
        a_ws = torch.full((k,), -1, dtype=torch.int32, device="cuda")
        nbytes = M.mbg_lm_head_workspace_size(k)
        ws = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
        M.mbg_lm_head(t, xd, k, l_ws, a_ws, ws, nbytes, s)
        l_na = torch.empty((k, V), dtype=torch.float32, device="cuda")
        a_na = torch.full((k,), -1, dtype=torch.int32, device="cuda")
        M.mbg_lm_head_noalloc(t, xd, k, l_na, a_na, s)
        torch.cuda.synchronize()
        g_ws, g_na = l_ws.cpu().numpy(), l_na.cpu().numpy()
        assert np.array_equal(g_ws, g_na), "logits differ from the workspace entry point"
        assert np.array_equal(a_ws.cpu().numpy(), a_na.cpu().numpy()), "argmax differs"
        ref = x.astype(np.float64) @ codecs.bf16_to_f64(w).T
        for j in range(k):
            compare_logits(g_na[j], ref[j], what=f"noalloc col {j}")
            check_argmax(int(a_na[j].item()), g_na[j], ref[j], what=f"noalloc col {j}")


def test_lm_head_noalloc_rejects_oversize_window():
    M = _M()
    w = torch.zeros((64, 256), dtype=torch.int16, device="cuda")
    x = torch.zeros((5, 256), dtype=torch.float32, device="cuda")
    a = torch.zeros(5, dtype=torch.int32, device="cuda")
    with pytest.raises(M.MbgError) as e:
        M.mbg_lm_head_noalloc(M.make_tensor(w, "bf16", 64, 256), x, 5, None, a, 0)
    assert e.value.code == M.MBG_E_RANGE
