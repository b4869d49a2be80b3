"""Shared helpers of the GPU tests: cached workload inputs and the tolerances.

Tolerances (scores, attention output) are those fixed for this path: scores
max-abs 1e-4 (float32) / 2e-2 (bf16); attention max-abs 1e-4 (float32), and for
bf16 max-abs 2e-2 together with mean-abs 2e-3.  Selected indices and gathered
rows must be bit-exact.
"""
import functools

import numpy as np
import pytest

from learned_token_pruning_scorer_amd import configs, inputs

SCORE_TOL = {"f32": 1e-4, "bf16": 2e-2}
ATTN_MAX_TOL = {"f32": 1e-4, "bf16": 2e-2}
ATTN_MEAN_TOL = {"f32": 1e-4, "bf16": 2e-3}


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from learned_token_pruning_scorer_amd import binding   # fails loudly if the library is missing
    return binding


@functools.lru_cache(maxsize=2)
def gate_inputs(name):
    return inputs.gate_inputs(configs.WORKLOADS[name])


def host_f64(t):
    """Device tensor -> exact float64 numpy."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy().astype(np.float64)


def log(msg):
    print(msg, flush=True)


# Gradients of the gated attention (dq, dk, dv, ds_kept): each element is judged against
# magnitudes of its own terms that the oracle reports (magnitudes=True), not against the
# tensor's largest value, so that one wrong row cannot hide under the heavy tail of the
# others.  A term carries a few bf16 roundings of 2^-8 relative error at most: the logit
# operands (the scaled query in bf16 moves P by about the logit's rounding), P and dZ
# packed to bf16 as MFMA operands, the forward's bf16 output inside D = rowsum(dout * out),
# and the bf16 result.  Two bounds per element:
#   worst case   |err| <= GRAD_C_SUM 2^-8 sum|terms|           (every rounding aligned)
#   statistical  |err| <= GRAD_C_RSS 2^-8 (rss(terms) + |ref|) (independent roundings add up
#                to about 2^-8 of the terms' root-sum-square; |ref| covers the result's own
#                rounding).  dk, dv and ds_kept sum over queries, whose operand roundings are
#                independent: 8 units.  dq sums over the keys of ONE query, and every term
#                shares that query's rounded operand, a common-mode error that grows with
#                the number of terms rather than its square root: 32 units.
# plus a floor for elements whose terms all vanish, and mean-abs <= 1e-2 mean|ref|.
GRAD_C_SUM = 4.0
GRAD_C_RSS = {"dq": 32.0, "dk": 8.0, "dv": 8.0, "ds_kept": 8.0}
GRAD_FLOOR = 1e-5


def grad_errors(got, ref, mag_sum, mag_rss):
    """(worst error in units of 2^-8 sum|terms|, worst in units of 2^-8 (rss + |ref|), mean-abs
    error, mean |ref|)."""
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    floor = GRAD_FLOOR * float(np.mean(mag_sum))
    w_sum = float(np.max(err / (2.0 ** -8 * mag_sum + floor / GRAD_C_SUM)))
    w_rss = float(np.max(err / (2.0 ** -8 * (mag_rss + np.abs(ref)) + floor / GRAD_C_SUM)))
    return w_sum, w_rss, float(err.mean()), float(np.abs(ref).mean())


def grad_within_bound(name, got, ref, mag_sum, mag_rss):
    """Both per-element bounds and the mean-abs bound hold for gradient `name` (and every
    element is finite)."""
    if not np.all(np.isfinite(got)):
        return False
    w_sum, w_rss, mean_err, mean_ref = grad_errors(got, ref, mag_sum, mag_rss)
    return w_sum <= GRAD_C_SUM and w_rss <= GRAD_C_RSS[name] and mean_err <= 1e-2 * mean_ref + 1e-6
