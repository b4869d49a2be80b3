"""The attention's precondition on the kept positions -- strictly increasing, as the
selection writes them (aiproducthub.cn, section 事件详情: kept tokens keep their order and
the causal mask is on original positions) -- checked by tg_check_positions, and enforced
by the debug build's attention entry points before they launch anything."""
import ctypes
import os

import numpy as np
import pytest

from learned_token_pruning_scorer_amd import inputs
from gpu_common import log, require_gpu

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "learned_token_pruning_scorer_amd", "libtokengate_debug.so")


@pytest.mark.parametrize("pos,bad", [
    ([0, 1, 2, 5, 9], 0), ([3], 0), ([], 0), ([0, 1, 1, 2], 1), ([5, 4, 3], 2), ([-1, 0, 1], 1),
    ([0, 2, 1, 3, 3, 2], 3),
])
def test_check_positions_counts_violations(pos, bad):
    binding = require_gpu()
    import torch
    t = torch.tensor(pos, dtype=torch.int32, device="cuda")
    assert int(binding.tg_check_positions(t).item()) == bad


def test_check_positions_large():
    binding = require_gpu()
    import torch
    g = np.random.default_rng(3)
    pos = np.sort(g.choice(10 ** 6, 100000, replace=False)).astype(np.int32)
    assert int(binding.tg_check_positions(torch.from_numpy(pos).cuda()).item()) == 0
    pos[5000] = pos[4999]
    pos[70000] = pos[69990]
    assert int(binding.tg_check_positions(torch.from_numpy(pos).cuda()).item()) == 2


def test_debug_build_rejects_unordered_positions():
    """The debug library's tg_gated_attention and tg_gated_attention_backward: TG_OK with the
    release library's output bits for ordered positions, TG_ERR_INVALID_ARG (nothing written)
    for unordered ones."""
    binding = require_gpu()
    import torch
    dbg = ctypes.CDLL(DEBUG_LIB)
    assert dbg.tg_debug_build() == 1
    p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    dbg.tg_gated_attention.restype = i32
    dbg.tg_gated_attention.argtypes = [i32, i64, i32, i32, i32, p, p, p, p, p, p, f32, p, p]
    g = np.random.default_rng(4)
    m, hq, hkv, d = 500, 8, 4, 128
    bf = lambda shape: binding.to_device(inputs.f32_to_bf16_bits(g.normal(size=shape).astype(np.float32)), "bf16")
    q, k, v = bf((m, hq, d)), bf((m, hkv, d)), bf((m, hkv, d))
    pos_np = np.sort(g.choice(5 * m, m, replace=False)).astype(np.int32)
    s = torch.from_numpy(g.normal(size=m).astype(np.float32)).cuda()
    gain = torch.from_numpy(g.uniform(0.5, 1.5, size=hq).astype(np.float32)).cuda()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = binding.tg_gated_attention(q, k, v, torch.from_numpy(pos_np).cuda(), s, gain, 1.1)
    out = torch.zeros_like(q)
    pos = torch.from_numpy(pos_np).cuda()
    assert dbg.tg_gated_attention(1, m, hq, hkv, d, ptr(q), ptr(k), ptr(v), ptr(pos), ptr(s), ptr(gain), 1.1, ptr(out),
                                  st) == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    bad = pos_np.copy()
    bad[[100, 101]] = bad[[101, 100]]
    posb = torch.from_numpy(bad).cuda()
    out2 = torch.zeros_like(q)
    log("[debug build] unordered positions are rejected")
    assert dbg.tg_gated_attention(1, m, hq, hkv, d, ptr(q), ptr(k), ptr(v), ptr(posb), ptr(s), ptr(gain), 1.1,
                                  ptr(out2), st) == 1
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out2.view(torch.int16))) == 0
