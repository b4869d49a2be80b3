"""tg_select_gather_noalloc -- the selection and gather with the library's static device
scratch instead of a caller workspace (for callers that cannot allocate) -- gives exactly
what tg_select_gather gives, on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents).  The selection keeps the K best document tokens
and the question (aiproducthub.cn, section 事件详情)."""
import ctypes

import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import inputs
from gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu


def _call_noalloc(binding, s, x, b, e, k, kept, xk, sk, status):
    import torch
    lib = binding.lib
    lib.tg_select_gather_noalloc.restype = ctypes.c_int32
    lib.tg_select_gather_noalloc.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.tg_select_gather_noalloc(1, s.shape[0], x.shape[1], p(s), b, e, k, p(x), x.stride(0), p(kept), p(xk),
                                        xk.stride(0), p(sk), p(status), st)


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_matches_workspace_entry_point(order):
    binding = require_gpu()
    import torch
    g = np.random.default_rng(77)
    cases = [(131072, 256, 0, 131008, 8192, g.normal(size=131072)),
             (5000, 64, 100, 4900, 333, np.round(g.normal(size=5000) * 4) / 4)]   # ties
    for n, d_model, b, e, k, s_np in cases:
        log(f"[select+gather noalloc] n={n} d_model={d_model} doc=[{b},{e}) k={k}")
        s = torch.from_numpy(s_np.astype(np.float32)).cuda()
        x_np = inputs.f32_to_bf16_bits(g.normal(size=(n, d_model)).astype(np.float32))
        x = binding.to_device(x_np, "bf16")
        m = binding.tg_num_kept(n, b, e, k)
        kept = torch.full((m,), -1, dtype=torch.int32, device="cuda")
        xk = torch.zeros(m, d_model, dtype=torch.bfloat16, device="cuda")
        sk = torch.zeros(m, dtype=torch.float32, device="cuda")
        status = torch.full((1,), 7, dtype=torch.int32, device="cuda")
        assert _call_noalloc(binding, s, x, b, e, k, kept, xk, sk, status) == 0
        ws = torch.zeros(binding.tg_select_workspace_bytes(n), dtype=torch.uint8, device="cuda")
        kept2, xk2, sk2 = binding.tg_select_gather(s, x, b, e, k, workspace=ws)
        binding.tg_select_check(ws)
        torch.cuda.synchronize()
        assert int(status.item()) == 0   # cleared by the call, no wait gave up
        assert torch.equal(kept, kept2)
        assert torch.equal(xk.view(torch.int16), xk2.view(torch.int16))
        assert torch.equal(sk.view(torch.int32), sk2.view(torch.int32))
        ref = oracle.select_topk(s_np.astype(np.float32).astype(np.float64), b, e, k)
        assert np.array_equal(kept.cpu().numpy().astype(np.int64), ref)
        assert np.array_equal(binding.to_host_bits(xk), x_np[ref])
