"""Several budgets in one launch and the random-K selector, against the oracle and the
single-budget call: every kept list must be bit-identical."""
import numpy as np
import pytest

import oracle
from gpu_common import gate_inputs, log, require_gpu
from learned_token_pruning_scorer_amd import configs

pytestmark = pytest.mark.gpu


def test_multi_budget_sweep_64k():
    binding = require_gpu()
    w = configs.WORKLOADS["sweep64k"]
    gi = gate_inputs("sweep64k")
    x = binding.to_device(gi.x, w.dtype)
    s = binding.tg_gate_score(x, binding.to_device(gi.w1, w.dtype), binding.to_device(gi.w2, w.dtype), None, gi.b2)
    log(f"[multi] sweep64k budgets {w.budgets}")
    lists = binding.tg_select_topk_multi(s, w.doc_begin, w.doc_end, w.budgets)
    s64 = s.cpu().numpy().astype(np.float64)
    for k, kept in zip(w.budgets, lists):
        one = binding.tg_select_topk(s, w.doc_begin, w.doc_end, k)
        assert np.array_equal(kept.cpu().numpy(), one.cpu().numpy())
        assert np.array_equal(kept.cpu().numpy(), oracle.select_topk(s64, w.doc_begin, w.doc_end, k))


@pytest.mark.parametrize("n,db,de,ks", [
    (1, 0, 1, [0, 1]),
    (3001, 500, 2500, [0, 1, 777, 1999, 2000, 5000, 3, 1000]),   # eight budgets, mixed modes
    (70000, 0, 69936, [1, 64, 4096, 30000]),                        # chunks larger than the register keys
    (5000, 2500, 2500, [7, 9]),                                     # empty document
    (140001, 1000, 139001, [0, 1, 4096, 8192, 65536, 138000, 200000, 17]),   # beyond the register keys
])
def test_multi_budget_edges(n, db, de, ks):
    binding = require_gpu()
    import torch
    g = np.random.default_rng(n + len(ks))
    s = np.round(g.normal(size=n), 2).astype(np.float32)   # ties
    s[g.choice(n, size=min(n, 5), replace=False)] = np.nan
    st = torch.from_numpy(s).cuda()
    log(f"[multi] n={n} doc=[{db},{de}) ks={ks}")
    lists = binding.tg_select_topk_multi(st, db, de, ks)
    for k, kept in zip(ks, lists):
        assert np.array_equal(kept.cpu().numpy(), oracle.select_topk(s.astype(np.float64), db, de, k))


@pytest.mark.parametrize("n,db,de,k,seed", [
    (1000, 0, 936, 100, 1), (1000, 0, 936, 100, 2), (131072, 0, 131008, 8192, 12345),
    (3001, 500, 2500, 0, 5), (3001, 500, 2500, 5000, 5), (70000, 64, 69000, 12345, 2**63 + 11),
    (140001, 7, 139999, 70000, 99),
])
def test_random_selector_matches_oracle(n, db, de, k, seed):
    binding = require_gpu()
    log(f"[random] n={n} doc=[{db},{de}) k={k} seed={seed}")
    kept = binding.tg_select_random(n, db, de, k, seed)
    assert np.array_equal(kept.cpu().numpy(), oracle.select_random(n, db, de, k, seed))


def test_random_selector_is_deterministic_and_seeded():
    binding = require_gpu()
    a = binding.tg_select_random(20000, 0, 19000, 500, 42).cpu().numpy()
    b = binding.tg_select_random(20000, 0, 19000, 500, 42).cpu().numpy()
    c = binding.tg_select_random(20000, 0, 19000, 500, 43).cpu().numpy()
    assert np.array_equal(a, b) and not np.array_equal(a, c)
