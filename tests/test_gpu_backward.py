"""Gradient of the token-gated attention on the GPU against the float64 oracle.

The backward path is the one by which a loss reaches the gate through the score
bias and trains the per-head gain and the temperature (aiproducthub.cn, section
事件详情; aisight.pl, section "Jak to dziala").  The oracle's gradient is pinned
on the CPU against torch autograd and finite differences.

Tolerances (bf16 operands, float32 accumulation, bf16 dq/dk/dv):
  dq, dk, dv, ds_kept   per element |err| <= 4 x 2^-8 sum|terms| and <= 32 x 2^-8 (rss(terms)
                        + |ref|), plus a floor, where the sum of the absolute values and the
                        root-sum-square of that element's terms come from the oracle
                        (magnitudes=True); and mean-abs <= 1e-2 mean|ref| + 1e-6
  dgain[h], dtau        |err| <= 2e-2 of the same sum over absolute terms, + 1e-4
A term carries a few bf16 roundings of 2^-8 each (the scaled query operand, P and dZ
packed as MFMA operands, the forward's bf16 output inside D, the bf16 result), so its
error is a small multiple of 2^-8 of its size: four of them bound the sum of the terms'
errors when every rounding aligns, and independent roundings add up to about 2^-8 of the
terms' root-sum-square, with a margin for the query operand's rounding that all terms of a
row share (gpu_common.py).  dgain and dtau are sums whose terms cancel (each row of
dZ sums to zero), so their error is judged against the sum of the terms' magnitudes,
not against the (possibly tiny) result; the absolute floors cover float32 rounding of
results that are exactly zero (a single visible key gives dZ = 0).
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import inputs
from gpu_common import GRAD_C_RSS, GRAD_C_SUM, grad_errors, grad_within_bound, host_f64, log, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # m, hq, hkv, d, bias, gapped positions ("top": gapped, near the int32 limit)
    (1, 4, 2, 64, True, False),
    (37, 4, 4, 64, True, True),
    (100, 8, 2, 128, True, False),
    (257, 8, 1, 64, False, True),
    (333, 16, 8, 128, True, True),
    (600, 6, 3, 64, True, False),
    (1088, 16, 8, 128, True, False),   # the 16k needle workload's kept rows (1024 + 64 question)
    (4224, 16, 8, 128, True, False),   # the 32k multi-document workload's kept rows (4096 + 128)
    (200, 4, 2, 128, True, "top"),     # positions within 10^6 of the int32 limit
]


def _case_inputs(m, hq, hkv, d, gapped, seed):
    g = np.random.default_rng(seed)
    bf = lambda shape: inputs.f32_to_bf16_bits(g.normal(size=shape).astype(np.float32))
    q, k, v, dout = bf((m, hq, d)), bf((m, hkv, d)), bf((m, hkv, d)), bf((m, hq, d))
    if gapped == "top":
        pos = np.sort(g.choice(np.arange(2**31 - 10**6, 2**31 - 1), m, replace=False)).astype(np.int32)
    else:
        pos = (np.sort(g.choice(5 * m + 3, m, replace=False)) if gapped else np.arange(m)).astype(np.int32)
    s = (g.normal(size=m) * 2).astype(np.float32)
    gain = g.uniform(0.5, 1.5, size=hq).astype(np.float32)
    return q, k, v, dout, pos, s, gain


def _run(binding, q, k, v, dout, pos, s, gain, tau, bias):
    import torch
    dev = "cuda"
    qt, kt, vt, dot = (binding.to_device(a, "bf16", dev) for a in (q, k, v, dout))
    pt = torch.from_numpy(pos).to(dev)
    st = torch.from_numpy(s).to(dev) if bias else None
    gt = torch.from_numpy(gain).to(dev) if bias else None
    out, lse = binding.tg_gated_attention_lse(qt, kt, vt, pt, st, gt, tau)
    grads = binding.tg_gated_attention_backward(qt, kt, vt, pt, st, gt, tau, out, lse, dot)
    torch.cuda.synchronize()
    return out, lse, grads


def _check_tensor(name, got, ref, mag):
    w_sum, w_rss, mean_err, mean_ref = grad_errors(got, ref, mag[name], mag[name + "_rss"])
    log(f"  {name}: worst |err| in 2^-8 sum|terms| {w_sum:.3f} (bound {GRAD_C_SUM}), in 2^-8 (rss + |ref|) "
        f"{w_rss:.3f} (bound {GRAD_C_RSS[name]}); mean_abs={mean_err:.3e} (|ref| mean {mean_ref:.3e}, "
        f"max {np.abs(ref).max():.3e})")
    assert grad_within_bound(name, got, ref, mag[name], mag[name + "_rss"]), name


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_matches_oracle(case):
    binding = require_gpu()
    m, hq, hkv, d, bias, gapped = case
    tau = 1.1
    q, k, v, dout, pos, s, gain = _case_inputs(m, hq, hkv, d, gapped, seed=m * 13 + hq + d)
    log(f"[attention backward] m={m} hq={hq} hkv={hkv} d={d} bias={bias} gapped={gapped}")
    out, lse, (dq, dk, dv, ds, dg, dtau) = _run(binding, q, k, v, dout, pos, s, gain, tau, bias)
    f64 = lambda a: inputs.to_f64(a, "bf16")
    ref = oracle.gated_attention_backward(f64(q), f64(k), f64(v), pos, s if bias else None,
                                          gain if bias else None, tau, f64(dout), magnitudes=True)
    rdq, rdk, rdv, rds, rdg, rdtau, mag = ref
    _check_tensor("dq", host_f64(dq), rdq, mag)
    _check_tensor("dk", host_f64(dk), rdk, mag)
    _check_tensor("dv", host_f64(dv), rdv, mag)
    if bias:
        _check_tensor("ds_kept", host_f64(ds), rds, mag)
        eg = np.abs(host_f64(dg) - rdg)
        log(f"  dgain: max_err/magnitude={np.max(eg / np.maximum(mag['dgain'], 1e-30)):.3e}")
        assert np.all(eg <= 2e-2 * mag["dgain"] + 1e-4)
    else:
        assert ds is None and dg is None
    et = abs(float(host_f64(dtau)[0]) - rdtau)
    log(f"  dtau: got {float(host_f64(dtau)[0]):.6e} ref {rdtau:.6e} magnitude {mag['dtau']:.3e}")
    assert et <= 2e-2 * mag["dtau"] + 1e-4

    rlse = oracle.gated_attention_lse(f64(q), f64(k), f64(v), pos, s if bias else None, gain if bias else None, tau)
    lerr = np.abs(host_f64(lse) - rlse)
    log(f"  lse: max_abs={lerr.max():.3e}")
    assert lerr.max() <= 2e-2


def test_backward_at_the_128k_workload_size_on_sampled_rows():
    """M = 8256 (the 128k workload's kept rows), Hq 16, Hkv 8, d 128, bias on, gapped positions,
    in the launch configuration the benchmark times.  The whole gradient is out of the
    oracle's reach at this size, so: the GPU's output and log-sum-exp on 64 sampled query rows
    against the oracle's, then dq on those rows and dk, dv, ds_kept on 64 sampled key rows
    against the oracle's per-row gradient fed the GPU's output and log-sum-exp (each stage
    checked on its own upstream, as for the forward)."""
    binding = require_gpu()
    m, hq, hkv, d = 8256, 16, 8, 128
    tau = 1.1
    q, k, v, dout, pos, s, gain = _case_inputs(m, hq, hkv, d, True, seed=128)
    log(f"[attention backward, sampled rows] m={m} hq={hq} hkv={hkv} d={d}")
    out, lse, (dq, dk, dv, ds, _, _) = _run(binding, q, k, v, dout, pos, s, gain, tau, True)
    qr = inputs.sample_rows(m, 64, forced=(0, m - 1), seed=3)
    kr = inputs.sample_rows(m, 64, forced=(0, m - 1), seed=4)
    f64 = lambda a: inputs.to_f64(a, "bf16")
    Q, K, V, dO = f64(q), f64(k), f64(v), f64(dout)
    o_gpu, l_gpu = host_f64(out), host_f64(lse)
    ro = oracle.gated_attention(Q, K, V, pos, s, gain, tau, rows=qr)
    eo = np.abs(o_gpu[qr] - ro)
    log(f"  out: max_abs={eo.max():.3e} mean_abs={eo.mean():.3e}")
    assert eo.max() <= 2e-2 and eo.mean() <= 2e-3
    el = np.abs(l_gpu[qr] - oracle.gated_attention_lse(Q, K, V, pos, s, gain, tau, rows=qr))
    log(f"  lse: max_abs={el.max():.3e}")
    assert el.max() <= 2e-2
    rq, rk, rv, rs, mag = oracle.gated_attention_backward_rows(Q, K, V, pos, s, gain, tau, dO, o_gpu, l_gpu, qr,
                                                               kr, magnitudes=True)
    _check_tensor("dq", host_f64(dq)[qr], rq, mag)
    _check_tensor("dk", host_f64(dk)[kr], rk, mag)
    _check_tensor("dv", host_f64(dv)[kr], rv, mag)
    _check_tensor("ds_kept", host_f64(ds)[kr], rs, mag)


def test_lse_variant_leaves_the_output_unchanged():
    """tg_gated_attention_lse writes the same output bits as tg_gated_attention."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d = 700, 8, 4, 128
    q, k, v, _, pos, s, gain = _case_inputs(m, hq, hkv, d, True, seed=5)
    qt, kt, vt = (binding.to_device(a, "bf16") for a in (q, k, v))
    pt, st, gt = (torch.from_numpy(a).cuda() for a in (pos, s, gain))
    o1 = binding.tg_gated_attention(qt, kt, vt, pt, st, gt, 0.8)
    o2, _ = binding.tg_gated_attention_lse(qt, kt, vt, pt, st, gt, 0.8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_backward_is_deterministic():
    """Fixed-order reductions: two calls give the same bits."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d = 1500, 16, 8, 128
    q, k, v, dout, pos, s, gain = _case_inputs(m, hq, hkv, d, False, seed=9)
    _, _, g1 = _run(binding, q, k, v, dout, pos, s, gain, 1.3, True)
    _, _, g2 = _run(binding, q, k, v, dout, pos, s, gain, 1.3, True)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_backward_zero_upstream_gradient():
    """dout = 0 gives exactly zero gradients everywhere."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d = 300, 8, 2, 64
    q, k, v, dout, pos, s, gain = _case_inputs(m, hq, hkv, d, False, seed=3)
    _, _, grads = _run(binding, q, k, v, np.zeros_like(dout), pos, s, gain, 1.0, True)
    for t in grads:
        assert torch.count_nonzero(t.float()) == 0


def test_backward_without_positions():
    """pos = NULL means pos = row index (the unpruned layout), also in the backward."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d, tau = 300, 8, 4, 128, 0.9
    q, k, v, dout, _, s, gain = _case_inputs(m, hq, hkv, d, False, seed=21)
    qt, kt, vt, dot = (binding.to_device(a, "bf16") for a in (q, k, v, dout))
    st, gt = torch.from_numpy(s).cuda(), torch.from_numpy(gain).cuda()
    out, lse = binding.tg_gated_attention_lse(qt, kt, vt, None, st, gt, tau)
    dq, dk, dv, ds, dg, dtau = binding.tg_gated_attention_backward(qt, kt, vt, None, st, gt, tau, out, lse, dot)
    torch.cuda.synchronize()
    f64 = lambda a: inputs.to_f64(a, "bf16")
    rdq, rdk, rdv, rds, rdg, rdtau, mag = oracle.gated_attention_backward(
        f64(q), f64(k), f64(v), np.arange(m), s, gain, tau, f64(dout), magnitudes=True)
    _check_tensor("dq", host_f64(dq), rdq, mag)
    _check_tensor("dk", host_f64(dk), rdk, mag)
    _check_tensor("dv", host_f64(dv), rdv, mag)
    _check_tensor("ds_kept", host_f64(ds), rds, mag)
    assert np.all(np.abs(host_f64(dg) - rdg) <= 2e-2 * mag["dgain"] + 1e-4)
    assert abs(float(host_f64(dtau)[0]) - rdtau) <= 2e-2 * mag["dtau"] + 1e-4
