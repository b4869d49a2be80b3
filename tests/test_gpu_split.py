"""Gated attention with the library's launch plan (tg_gated_attention_split) on the GPU
against the oracle.

The variant computes the same logits and mask as tg_gated_attention (aiproducthub.cn,
section 事件详情; aisight.pl, section "Jak to dziala"), with each long query tile's keys
walked by two groups of waves, or cut into runs over workgroups, whose partial softmax
states are merged.  Its output is judged with the
attention tolerances (bf16: max-abs 2e-2, mean-abs 2e-3); the runs' normalised rows are
kept in float32.  The lse merge adds only float32
rounding to the unsplit kernel's arithmetic, so the lse is held to the backward
test's 2e-2 and, against the unsplit kernel's own lse, to 2^-7: each side's row sum adds
P values rounded to bf16 (unit roundoff 2^-8) against its own running max, so each log
row sum lies within 2^-8 of the one of the unrounded P, and the two within 2^-7.
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import inputs
from gpu_common import ATTN_MAX_TOL, ATTN_MEAN_TOL, grad_errors, grad_within_bound, host_f64, log, require_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # m, hq, hkv, d, bias, gapped positions, split_tiles
    (130, 4, 2, 64, True, False, 1),       # runs of one key tile
    (300, 8, 1, 128, True, True, 2),       # 4 heads per workgroup, 32-row query tiles
    (517, 6, 6, 64, False, False, 3),      # 128-row query tiles: some waves see no key of a run
    (777, 3, 1, 128, True, True, 5),       # odd group, ragged last tile
    (1088, 16, 8, 128, True, True, 0),     # the 16k needle workload's kept rows: key groups
    (2112, 16, 8, 128, True, False, 0),    # 64k sweep, K = 2048: key groups
    (1088, 16, 8, 128, True, True, 4),     # runs of 4 forced
    (2112, 2, 1, 128, True, True, 0),      # one head slot: automatic runs of 8
    (1000, 4, 2, 64, True, False, 0),      # two head slots: automatic runs
    (64, 4, 2, 64, True, False, 1),        # one query tile: no split at all
    (1, 16, 8, 128, True, False, 0),
]


def _inputs(m, hq, hkv, d, gapped, seed):
    g = np.random.default_rng(seed)
    q, k, v = (inputs.f32_to_bf16_bits(g.normal(size=(m, h, d)).astype(np.float32)) for h in (hq, hkv, hkv))
    pos = (np.sort(g.choice(5 * m + 3, m, replace=False)) if gapped else np.arange(m)).astype(np.int32)
    s = (g.normal(size=m) * 2).astype(np.float32)
    gain = g.uniform(0.5, 1.5, size=hq).astype(np.float32)
    return q, k, v, pos, s, gain


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_split_attention_matches_oracle(case):
    binding = require_gpu()
    import torch
    m, hq, hkv, d, bias, gapped, split = case
    q, k, v, pos, s, gain = _inputs(m, hq, hkv, d, gapped, seed=m * 13 + hq + split)
    tau = 1.1
    need = binding.tg_gated_attention_split_workspace_bytes(m, hq, hkv, d, split)
    log(f"[split attention] m={m} hq={hq} hkv={hkv} d={d} bias={bias} gapped={gapped} split={split} ws={need}")
    qt, kt, vt = (binding.to_device(a, "bf16") for a in (q, k, v))
    pt = torch.from_numpy(pos).cuda()
    st = torch.from_numpy(s).cuda() if bias else None
    gt = torch.from_numpy(gain).cuda() if bias else None
    lse = torch.empty(m, hq, dtype=torch.float32, device="cuda")
    o = binding.tg_gated_attention_split(qt, kt, vt, pt, st, gt, tau, lse=lse, split_tiles=split)
    o_plain, lse_plain = binding.tg_gated_attention_lse(qt, kt, vt, pt, st, gt, tau)
    torch.cuda.synchronize()
    rows = np.arange(m) if m <= 1100 else inputs.sample_rows(m, 256, forced=(0, m - 1), seed=1)
    f64 = lambda a: inputs.to_f64(a, "bf16")
    ref = oracle.gated_attention(f64(q), f64(k), f64(v), pos, s if bias else None, gain if bias else None, tau,
                                 rows=rows)
    err = np.abs(host_f64(o)[rows] - ref)
    log(f"  out: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= ATTN_MAX_TOL["bf16"] and err.mean() <= ATTN_MEAN_TOL["bf16"]
    if m <= 1100:
        rlse = oracle.gated_attention_lse(f64(q), f64(k), f64(v), pos, s if bias else None,
                                          gain if bias else None, tau)
        lerr = np.abs(host_f64(lse) - rlse)
        log(f"  lse: max_abs={lerr.max():.3e}")
        assert lerr.max() <= 2e-2
    dl = np.abs(host_f64(lse) - host_f64(lse_plain))
    log(f"  against the unsplit kernel: out max_abs={np.abs(host_f64(o) - host_f64(o_plain)).max():.3e} "
        f"lse max_abs={dl.max():.3e}")
    assert dl.max() <= 2.0 ** -7
    if need == 0:   # no split: the very same kernel as the unsplit entry point
        assert torch.equal(o, o_plain) and torch.equal(lse, lse_plain)


def test_split_attention_is_deterministic_and_reuses_its_workspace():
    """Two calls give the same bits; a workspace left dirty by a larger call is fine."""
    binding = require_gpu()
    import torch
    big = _inputs(2112, 16, 8, 128, False, seed=3)
    small = _inputs(1088, 16, 8, 128, True, seed=4)
    need = binding.tg_gated_attention_split_workspace_bytes(2112, 16, 8, 128, 3)
    assert need >= binding.tg_gated_attention_split_workspace_bytes(1088, 16, 8, 128, 3) > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    outs = []
    for q, k, v, pos, s, gain in (big, small, small):
        qt, kt, vt = (binding.to_device(a, "bf16") for a in (q, k, v))
        pt, st, gt = (torch.from_numpy(a).cuda() for a in (pos, s, gain))
        outs.append(binding.tg_gated_attention_split(qt, kt, vt, pt, st, gt, 0.9, split_tiles=3, workspace=ws))
    torch.cuda.synchronize()
    assert torch.equal(outs[1], outs[2])
    q, k, v, pos, s, gain = small
    ref = oracle.gated_attention(*(inputs.to_f64(a, "bf16") for a in (q, k, v)), pos, s, gain, 0.9)
    err = np.abs(host_f64(outs[1]) - ref)
    assert err.max() <= ATTN_MAX_TOL["bf16"] and err.mean() <= ATTN_MEAN_TOL["bf16"]


def test_backward_from_split_forward():
    """The split forward's out and lse feed the backward like the unsplit ones."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d = 1088, 16, 8, 128
    q, k, v, pos, s, gain = _inputs(m, hq, hkv, d, False, seed=8)
    dout = inputs.f32_to_bf16_bits(np.random.default_rng(9).normal(size=(m, hq, d)).astype(np.float32))
    qt, kt, vt, dt = (binding.to_device(a, "bf16") for a in (q, k, v, dout))
    pt, st, gt = (torch.from_numpy(a).cuda() for a in (pos, s, gain))
    lse = torch.empty(m, hq, dtype=torch.float32, device="cuda")
    out = binding.tg_gated_attention_split(qt, kt, vt, pt, st, gt, 1.2, lse=lse)
    dq, dk, dv, ds, dg, dtau = binding.tg_gated_attention_backward(qt, kt, vt, pt, st, gt, 1.2, out, lse, dt)
    torch.cuda.synchronize()
    f64 = lambda a: inputs.to_f64(a, "bf16")
    rdq, rdk, rdv, rds, _, _, mag = oracle.gated_attention_backward(f64(q), f64(k), f64(v), pos, s, gain, 1.2,
                                                                    f64(dout), magnitudes=True)
    for name, got, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("ds_kept", ds, rds)):
        w_sum, w_rss, mean_err, _ = grad_errors(host_f64(got), r, mag[name], mag[name + "_rss"])
        log(f"  {name}: worst |err| in 2^-8 sum|terms| {w_sum:.3f}, in 2^-8 (rss + |ref|) {w_rss:.3f}, "
            f"mean_abs={mean_err:.3e}")
        assert grad_within_bound(name, host_f64(got), r, mag[name], mag[name + "_rss"]), name
