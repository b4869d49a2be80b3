"""Kept-row projection + rotary embedding + KV emission on the GPU against the oracle.

Tolerance, element-wise: |gpu - ref| <= 2^-8 |ref| + 1e-5 rms(ref).  The exact value
rounded to bf16 is within 2^-8 |ref| (bf16's unit roundoff); float32 accumulation of
bf16 products over
d_model and the float32 rotation (cos / sin accurate to ~1e-7 after the float64 angle
reduction) add errors far below 1e-5 of the typical magnitude, including on outputs
that cancel to near zero.  Positions, the cache slots and untouched cache rows are
compared exactly.
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import configs, inputs
from gpu_common import ATTN_MAX_TOL, ATTN_MEAN_TOL, gate_inputs, host_f64, log, require_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F   # bf16 bits written into the caches first; rows outside the call's slots must keep them


def _check(name, got, ref):
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * rms
    worst = float(np.max(err / np.maximum(bound, 1e-30))) if ref.size else 0.0
    log(f"  {name}: max_abs={err.max() if err.size else 0:.3e} rms(ref)={rms:.3e} worst err/bound={worst:.3f}")
    assert np.all(err <= bound), name


CASES = [
    # m, d_model, hq, hkv, d, bias, slot0, extra capacity
    (1, 64, 2, 1, 64, False, 0, 0),
    (37, 128, 4, 2, 64, True, 5, 3),
    (70, 128, 1, 1, 128, True, 0, 0),       # 384 features: the last feature tile is half empty
    (300, 256, 4, 2, 128, False, 0, 10),
    (333, 192, 6, 1, 64, True, 17, 0),
    (517, 512, 16, 8, 128, True, 100, 83),
    # grids large enough for the XCD-blocked tile order: 8 feature tiles x 57 token tiles
    # (ragged last block), and 3 feature tiles (the last half empty) x 162 token tiles
    (14500, 64, 8, 4, 128, True, 11, 4),
    (41300, 64, 3, 1, 128, False, 0, 0),
    # 16 feature tiles x 16 full token tiles fill a 256-CU chip exactly, so the ragged last
    # token rows (64 and 100) go to the second launch of 128-token tiles
    (4160, 64, 16, 8, 128, True, 3, 2),
    (4196, 64, 32, 16, 64, False, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_qkv_rope_matches_oracle(case):
    binding = require_gpu()
    import torch
    m, d_model, hq, hkv, d, use_bias, slot0, extra = case
    g = np.random.default_rng(m * 31 + d_model + d)
    n_feat = (hq + 2 * hkv) * d
    x = inputs.f32_to_bf16_bits(g.normal(size=(m, d_model)).astype(np.float32))
    w = inputs.f32_to_bf16_bits((g.normal(size=(n_feat, d_model)) / np.sqrt(d_model)).astype(np.float32))
    b = (g.normal(size=n_feat) * 0.1).astype(np.float32) if use_bias else None
    pos = np.sort(g.choice(131072, m, replace=False)).astype(np.int32)
    theta = 1e6
    cap = slot0 + m + extra
    log(f"[qkv_rope] m={m} d_model={d_model} hq={hq} hkv={hkv} d={d} bias={use_bias} slot0={slot0} cap={cap}")
    dev = "cuda"
    kc = torch.full((cap, hkv, d), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    vc = torch.full((cap, hkv, d), SENTINEL, dtype=torch.int16, device=dev).view(torch.bfloat16)
    pc = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    q, kc, vc, pc = binding.tg_qkv_rope(
        binding.to_device(x, "bf16", dev), binding.to_device(w, "bf16", dev), torch.from_numpy(pos).to(dev),
        hq, hkv, d, theta, b_qkv=torch.from_numpy(b).to(dev) if use_bias else None,
        k_cache=kc, v_cache=vc, pos_cache=pc, cache_slot0=slot0)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope(inputs.to_f64(x, "bf16"), inputs.to_f64(w, "bf16"), b, hq, hkv, d, pos, theta)
    _check("q", host_f64(q), rq)
    _check("k", host_f64(kc[slot0:slot0 + m]), rk)
    _check("v", host_f64(vc[slot0:slot0 + m]), rv)
    pc_h = pc.cpu().numpy()
    np.testing.assert_array_equal(pc_h[slot0:slot0 + m], pos)
    outside = np.r_[0:slot0, slot0 + m:cap]
    assert np.all(pc_h[outside] == -7)
    for c in (kc, vc):
        bits = c.view(torch.int16).cpu().numpy()[outside]
        assert np.all(bits == SENTINEL)


def test_qkv_rope_at_the_128k_workload_size_on_sampled_rows():
    """M = 8256 kept rows of d_model 2048 to Hq 16 / Hkv 8 heads of 128, positions from a
    131072-token prompt, in the launch configuration the benchmark times; the projection is
    row-local, so the oracle computes 64 sampled rows (the first and last forced) on their own."""
    binding = require_gpu()
    import torch
    g = np.random.default_rng(8256)
    m, d_model, hq, hkv, d = 8256, 2048, 16, 8, 128
    n_feat = (hq + 2 * hkv) * d
    x = inputs.f32_to_bf16_bits(g.normal(size=(m, d_model)).astype(np.float32))
    w = inputs.f32_to_bf16_bits((g.normal(size=(n_feat, d_model)) / np.sqrt(d_model)).astype(np.float32))
    pos = np.sort(g.choice(131072, m, replace=False)).astype(np.int32)
    theta = 1e6
    log(f"[qkv_rope, sampled rows] m={m} d_model={d_model} hq={hq} hkv={hkv} d={d}")
    pc = torch.full((m,), -7, dtype=torch.int32, device="cuda")
    q, kc, vc, pc = binding.tg_qkv_rope(binding.to_device(x, "bf16"), binding.to_device(w, "bf16"),
                                        torch.from_numpy(pos).cuda(), hq, hkv, d, theta, pos_cache=pc)
    torch.cuda.synchronize()
    rows = inputs.sample_rows(m, 64, forced=(0, m - 1), seed=5)
    rq, rk, rv = oracle.qkv_rope(inputs.to_f64(x[rows], "bf16"), inputs.to_f64(w, "bf16"), None, hq, hkv, d,
                                 pos[rows], theta)
    _check("q", host_f64(q)[rows], rq)
    _check("k", host_f64(kc)[rows], rk)
    _check("v", host_f64(vc)[rows], rv)
    np.testing.assert_array_equal(pc.cpu().numpy(), pos)


def test_qkv_rope_without_position_cache_and_large_positions():
    """Positions near 2^31 (angles of ~2e9 rad) still rotate accurately."""
    binding = require_gpu()
    import torch
    g = np.random.default_rng(77)
    m, d_model, hq, hkv, d = 96, 128, 2, 1, 128
    n_feat = (hq + 2 * hkv) * d
    x = inputs.f32_to_bf16_bits(g.normal(size=(m, d_model)).astype(np.float32))
    w = inputs.f32_to_bf16_bits((g.normal(size=(n_feat, d_model)) / np.sqrt(d_model)).astype(np.float32))
    pos = np.sort(g.choice(np.arange(2**31 - 10**6, 2**31 - 1), m, replace=False)).astype(np.int32)
    q, kc, vc, _ = binding.tg_qkv_rope(binding.to_device(x, "bf16"), binding.to_device(w, "bf16"),
                                       torch.from_numpy(pos).cuda(), hq, hkv, d, 1e4)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_rope(inputs.to_f64(x, "bf16"), inputs.to_f64(w, "bf16"), None, hq, hkv, d, pos, 1e4)
    _check("q", host_f64(q), rq)
    _check("k", host_f64(kc), rk)
    _check("v", host_f64(vc), rv)


def test_kept_rows_to_attention_16k():
    """16k needle workload: select -> gather -> projection / rotary / KV emission -> gated
    attention reading K and V from the emitted cache, each stage against the oracle on the
    GPU's own upstream output."""
    binding = require_gpu()
    import torch
    w = configs.WORKLOADS["niah16k"]
    gi = gate_inputs("niah16k")
    k = w.budgets[0]
    dev = "cuda"
    x_t = binding.to_device(gi.x, w.dtype, dev)
    scores = binding.tg_gate_score(x_t, binding.to_device(gi.w1, w.dtype, dev), binding.to_device(gi.w2, w.dtype, dev),
                                   torch.from_numpy(gi.b1).to(dev), gi.b2)
    kept = binding.tg_select_topk(scores, w.doc_begin, w.doc_end, k)
    xk, sk = binding.tg_gather_kept(x_t, kept, scores)
    wq = inputs.qkv_weights(w)
    log(f"[niah16k kept rows -> qkv_rope -> attention] m={kept.numel()}")
    q, kc, vc, pc = binding.tg_qkv_rope(xk, binding.to_device(wq, w.dtype, dev), kept, w.n_q_heads, w.n_kv_heads,
                                        w.head_dim, inputs.ROPE_THETA,
                                        pos_cache=torch.empty(kept.numel(), dtype=torch.int32, device=dev))
    gain = torch.from_numpy(inputs.gains(w)).to(dev)
    o = binding.tg_gated_attention(q, kc, vc, pc, sk, gain, w.tau)
    torch.cuda.synchronize()
    kept_h = kept.cpu().numpy()
    assert np.array_equal(pc.cpu().numpy(), kept_h)
    rq, rk, rv = oracle.qkv_rope(host_f64(xk), inputs.to_f64(wq, w.dtype), None, w.n_q_heads, w.n_kv_heads,
                                 w.head_dim, kept_h, inputs.ROPE_THETA)
    _check("q", host_f64(q), rq)
    _check("k", host_f64(kc), rk)
    _check("v", host_f64(vc), rv)
    m = kept.numel()
    rows = inputs.sample_rows(m, 256, forced=(0, m - 1, inputs.first_question_row(w, k)), seed=3)
    ref = oracle.gated_attention(host_f64(q), host_f64(kc), host_f64(vc), kept_h, host_f64(sk), host_f64(gain),
                                 w.tau, rows=rows)
    err = np.abs(host_f64(o)[rows] - ref)
    log(f"  attention on emitted K/V: rows={len(rows)} max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= ATTN_MAX_TOL["bf16"] and err.mean() <= ATTN_MEAN_TOL["bf16"]
