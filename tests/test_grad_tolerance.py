"""The per-element gradient bounds of the GPU backward tests (gpu_common.grad_within_bound),
checked on the CPU: they accept the oracle's gradient rounded to bf16 (what the GPU's
outputs carry at the least), and they reject a gradient with a single wrong key or query
row -- wrong rows that the earlier bound, relative to the tensor's largest element, let
through.  The gradient is that of the token-gated attention (aiproducthub.cn, section
事件详情: the score bias is the scorer's gradient path)."""
import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import inputs
from gpu_common import grad_within_bound

NAMES = ["dq", "dk", "dv", "ds_kept"]


def _bf16_round(a):
    return inputs.to_f64(inputs.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)), "bf16")


@pytest.fixture(scope="module")
def grads():
    g = np.random.default_rng(7)
    m, hq, hkv, d = 300, 8, 4, 64
    bf = lambda shape: inputs.to_f64(inputs.f32_to_bf16_bits(g.normal(size=shape).astype(np.float32)), "bf16")
    q, k, v, dout = bf((m, hq, d)), bf((m, hkv, d)), bf((m, hkv, d)), bf((m, hq, d))
    pos = np.arange(m)
    s = g.normal(size=m) * 2
    gain = g.uniform(0.5, 1.5, size=hq)
    res = oracle.gated_attention_backward(q, k, v, pos, s, gain, 1.1, dout, magnitudes=True)
    return dict(zip(NAMES, res[:4])), res[6]


def _old_bound(got, ref):
    """The earlier bound: max-abs relative to the tensor's largest element, plus the mean."""
    err = np.abs(got - ref)
    return err.max() <= 3e-2 * np.abs(ref).max() + 1e-5 and err.mean() <= 1e-2 * np.abs(ref).mean() + 1e-6


@pytest.mark.parametrize("name", NAMES)
def test_bound_accepts_bf16_rounding(grads, name):
    ref, mag = grads[0][name], grads[1]
    assert grad_within_bound(name, _bf16_round(ref), ref, mag[name], mag[name + "_rss"])


@pytest.mark.parametrize("name", NAMES)
def test_bound_rejects_one_wrong_row(grads, name):
    """Row r replaced by its neighbour's (an off-by-one in a tile's row index).  Among the
    rows where the earlier bound accepts that mistake, the new bounds reject most, and the
    one with the largest error against the tensor's largest element."""
    ref, mag = grads[0][name], grads[1]
    flat = ref.reshape(ref.shape[0], -1)
    passed_old, rejected = [], []
    for r in range(ref.shape[0] - 1):
        bad = ref.copy()
        bad[r] = ref[r + 1]
        bad = _bf16_round(bad)
        if _old_bound(bad, ref):
            passed_old.append((float(np.abs(flat[r] - flat[r + 1]).max()), r))
            rejected.append(not grad_within_bound(name, bad, ref, mag[name], mag[name + "_rss"]))
    if name == "dq":
        # dq's rows are not heavy-tailed here: the earlier bound already rejects them all,
        # and so does the new one
        assert not passed_old
        for r in (0, 150, ref.shape[0] - 2):
            bad = ref.copy()
            bad[r] = ref[r + 1]
            assert not grad_within_bound(name, _bf16_round(bad), ref, mag[name], mag[name + "_rss"])
        return
    # ds_kept's neighbours are close now and then (a key's ds is a random sum of the size of
    # its terms' root-sum-square), so a few swaps stay inside the rounding bound there
    assert np.mean(rejected) >= (0.8 if name == "ds_kept" else 0.95)
    worst = max(passed_old)[1]
    assert rejected[[r for _, r in passed_old].index(worst)]


def test_bound_rejects_a_short_key_row(grads):
    """dk of one key 10% short (e.g. one query tile's contribution dropped)."""
    ref, mag = grads[0]["dk"], grads[1]
    bad = ref.copy()
    bad[100] *= 0.9
    assert _old_bound(_bf16_round(bad), ref)
    assert not grad_within_bound("dk", _bf16_round(bad), ref, mag["dk"], mag["dk_rss"])
