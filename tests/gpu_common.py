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
