"""Pins of the float64 oracle against things other than itself.

Each check uses an independent source: tabulated normal-CDF values, torch's own
GELU / Linear / scaled_dot_product_attention in float64, brute-force full sorts,
a scalar textbook attention loop, and invariants of the definitions.  The cases
are chosen so that a dropped term (bias, gain, temperature, b1, b2), a wrong sign,
a wrong head mapping or a transposed operand fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _table(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "normal_cdf.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, p = line.split()
                rows.append((float(x), float(p)))
    return rows


# --------------------------------------------------------------------------- GELU
def test_gelu_matches_tabulated_normal_cdf(golden_dir):
    for x, phi in _table(golden_dir):
        assert oracle.gelu(x) == pytest.approx(x * phi, abs=1e-15)
        assert oracle.gelu(-x) == pytest.approx(-x * (1.0 - phi), abs=1e-15)


def test_gelu_matches_torch_exact_gelu_and_ndtr():
    x = np.random.default_rng(1).normal(scale=4.0, size=2000)
    xt = torch.from_numpy(x)
    ref = torch.nn.functional.gelu(xt, approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(x), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.gelu(x), (xt * torch.special.ndtr(xt)).numpy(), rtol=0, atol=1e-13)


def test_gelu_limits_and_odd_part():
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu(40.0) == 40.0
    assert abs(oracle.gelu(-40.0)) < 1e-300
    x = np.linspace(-6, 6, 97)
    # GELU(x) - GELU(-x) = x  (Phi(x) + Phi(-x) = 1)
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, atol=1e-14)


# --------------------------------------------------------------------------- scorer
def test_gate_score_matches_torch_mlp():
    g = np.random.default_rng(2)
    n, d, h = 37, 24, 10
    x = g.normal(size=(n, d))
    w1 = g.normal(size=(h, d)) / math.sqrt(d)
    b1 = g.normal(size=h)
    w2 = g.normal(size=h)
    b2 = 0.37
    lin1 = torch.nn.Linear(d, h, dtype=torch.float64)
    lin2 = torch.nn.Linear(h, 1, dtype=torch.float64)
    with torch.no_grad():
        lin1.weight.copy_(torch.from_numpy(w1))
        lin1.bias.copy_(torch.from_numpy(b1))
        lin2.weight.copy_(torch.from_numpy(w2[None, :]))
        lin2.bias.fill_(b2)
        ref = lin2(torch.nn.GELU()(lin1(torch.from_numpy(x))))[:, 0].numpy()
    np.testing.assert_allclose(oracle.gate_score(x, w1, b1, w2, b2), ref, rtol=0, atol=1e-12)


def test_gate_score_one_hot_reads_table_values(golden_dir):
    # w1 row j is the unit vector e_{perm[j]} (non-square: d_model=6, d_hidden=4),
    # so h[i, j] = x[i, perm[j]] + b1[j]; w2 = e_j2 picks one hidden unit.
    table = [(x, p) for x, p in _table(golden_dir) if x > 0]
    perm = [4, 0, 5, 2]
    d, hdim = 6, 4
    w1 = np.zeros((hdim, d))
    for j, c in enumerate(perm):
        w1[j, c] = 1.0
    b1 = np.array([0.25, -0.5, 0.5, 1.0])
    b2 = -0.125
    j2 = 2                           # hidden unit 2 reads column 5, bias +0.5
    w2 = np.zeros(hdim)
    w2[j2] = 1.0
    x = np.zeros((len(table), d))
    for i, (xv, _) in enumerate(table):
        x[i, perm[j2]] = xv - b1[j2]          # h = xv exactly
        x[i, perm[0]] = 7.0                   # other units must not leak in
    s = oracle.gate_score(x, w1, b1, w2, b2)
    expect = np.array([xv * p for xv, p in table]) + b2
    np.testing.assert_allclose(s, expect, rtol=0, atol=1e-15)
    # negative side: h = -xv -> GELU = -xv * (1 - Phi(xv))
    x2 = np.zeros((len(table), d))
    for i, (xv, _) in enumerate(table):
        x2[i, perm[j2]] = -xv - b1[j2]
    s2 = oracle.gate_score(x2, w1, b1, w2, 0.0)
    np.testing.assert_allclose(s2, np.array([-xv * (1 - p) for xv, p in table]), rtol=0, atol=1e-15)


def test_gate_score_linear_in_w2_and_b2():
    g = np.random.default_rng(3)
    x = g.normal(size=(9, 8)); w1 = g.normal(size=(5, 8))
    wa, wb = g.normal(size=5), g.normal(size=5)
    sa = oracle.gate_score(x, w1, None, wa, 0.0)
    sb = oracle.gate_score(x, w1, None, wb, 0.0)
    np.testing.assert_allclose(oracle.gate_score(x, w1, None, 2 * wa - 3 * wb, 1.5), 2 * sa - 3 * sb + 1.5,
                               atol=1e-12)


# --------------------------------------------------------------------------- selection
def _brute_force(s, b, e, k):
    """Full sort of the document by (score desc, position asc), NaN last."""
    doc = list(range(b, e))
    def key(i):
        v = s[i]
        return (1, 0.0, i) if math.isnan(v) else (0, -v, i)
    top = sorted(doc, key=key)[:min(k, e - b)]
    return sorted(set(range(0, b)) | set(range(e, len(s))) | set(top))


def _random_scores(g, n):
    kind = g.integers(0, 4)
    if kind == 0:
        return g.normal(size=n)
    if kind == 1:       # heavy ties
        return g.integers(-3, 4, size=n).astype(np.float64)
    if kind == 2:       # signed zeros, infinities and NaNs mixed with ties
        pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5])
        return pool[g.integers(0, len(pool), size=n)]
    return np.full(n, 0.5)  # all equal


@pytest.mark.parametrize("seed", range(60))
def test_select_matches_brute_force_sort(seed):
    g = np.random.default_rng(100 + seed)
    n = int(g.integers(1, 40))
    b = int(g.integers(0, n + 1)); e = int(g.integers(b, n + 1))
    s = _random_scores(g, n)
    d = e - b
    for k in sorted({0, 1, max(d - 1, 0), d, d + 5, int(g.integers(0, d + 1))}):
        got = oracle.select_topk(s, b, e, k)
        assert got.tolist() == _brute_force(s, b, e, k), (s, b, e, k)
        assert len(got) == oracle.num_kept(n, b, e, k)


def test_select_invariants_on_tiny_workload():
    from learned_token_pruning_scorer_amd import configs, inputs
    w = configs.WORKLOADS["tiny"]
    gi = inputs.gate_inputs(w)
    s = oracle.gate_score(inputs.to_f64(gi.x, w.dtype), inputs.to_f64(gi.w1, w.dtype), gi.b1,
                          inputs.to_f64(gi.w2, w.dtype), gi.b2)
    k = w.budgets[0]
    kept = oracle.select_topk(s, w.doc_begin, w.doc_end, k)
    assert len(kept) == w.n_kept(k)
    assert np.all(np.diff(kept) > 0)
    doc_kept = kept[(kept >= w.doc_begin) & (kept < w.doc_end)]
    assert len(doc_kept) == min(k, w.n_doc)
    assert set(range(w.doc_end, w.n)) <= set(kept.tolist())
    dropped = np.setdiff1d(np.arange(w.doc_begin, w.doc_end), doc_kept)
    assert s[doc_kept].min() >= s[dropped].max()
    t = s[doc_kept].min()
    tied_kept, tied_dropped = doc_kept[s[doc_kept] == t], dropped[s[dropped] == t]
    if len(tied_dropped):
        assert tied_kept.max() < tied_dropped.min()


@pytest.mark.parametrize("seed", range(8))
def test_select_nested_across_budgets(seed):
    g = np.random.default_rng(200 + seed)
    n = 300
    s = g.integers(-20, 20, size=n).astype(np.float64) / 4.0
    prev = set(oracle.select_topk(s, 10, 280, 0).tolist())
    for k in range(1, 275, 7):
        cur = set(oracle.select_topk(s, 10, 280, k).tolist())
        assert prev <= cur
        prev = cur


def test_select_rejects_bad_spans():
    with pytest.raises(ValueError):
        oracle.select_topk(np.zeros(4), 3, 2, 1)
    with pytest.raises(ValueError):
        oracle.select_topk(np.zeros(4), 0, 5, 1)
    with pytest.raises(ValueError):
        oracle.select_topk(np.zeros(4), 0, 4, -1)


# --------------------------------------------------------------------------- gather
def test_gather_is_row_indexing():
    g = np.random.default_rng(4)
    x = g.normal(size=(11, 3)); s = g.normal(size=11)
    kept = np.array([0, 2, 3, 7, 10])
    xk, sk = oracle.gather_kept(x, s, kept)
    assert xk.tolist() == [x[i].tolist() for i in kept]
    assert sk.tolist() == [s[i] for i in kept]


# --------------------------------------------------------------------------- attention
def _sdpa_reference(q, k, v, pos, s_kept, gain, tau):
    """torch SDPA in float64 with an additive mask = bias + causal(-inf on positions)."""
    m, hq, d = q.shape
    group = hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, M, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    pos_t = torch.from_numpy(np.asarray(pos, dtype=np.int64))
    mask = torch.zeros(hq, m, m, dtype=torch.float64)
    if s_kept is not None:
        mask += torch.from_numpy(np.asarray(gain, np.float64))[:, None, None] * \
            torch.from_numpy(np.asarray(s_kept, np.float64))[None, None, :]
    mask = mask.masked_fill(pos_t[None, :] > pos_t[:, None], float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=mask, scale=1.0 / (math.sqrt(d) * tau))
    return out.permute(1, 0, 2).numpy()


def _attn_case(seed, m=37, hq=4, hkv=2, d=16):
    g = np.random.default_rng(seed)
    q = g.normal(size=(m, hq, d)); k = g.normal(size=(m, hkv, d)); v = g.normal(size=(m, hkv, d))
    s = g.normal(size=m) * 2.0
    gain = g.uniform(0.5, 1.5, size=hq)
    pos = np.sort(g.choice(4 * m, size=m, replace=False))
    return q, k, v, pos, s, gain


@pytest.mark.parametrize("hq,hkv", [(4, 2), (4, 4), (6, 2), (3, 1)])
def test_attention_matches_torch_sdpa_with_bias_mask(hq, hkv):
    q, k, v, pos, s, gain = _attn_case(5 + hq + hkv, hq=hq, hkv=hkv)
    tau = 1.3
    got = oracle.gated_attention(q, k, v, pos, s, gain, tau)
    ref = _sdpa_reference(q, k, v, pos, s, gain, tau)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_unbiased_tau1_is_textbook_causal_sdpa():
    q, k, v, _, _, _ = _attn_case(6)
    m, hq, d = q.shape
    got = oracle.causal_attention(q, k, v)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(2, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(2, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), kt, vt, is_causal=True).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_scalar_loop_tiny():
    # scalar textbook evaluation: M=5, Hq=2, Hkv=1, d=3, gapped positions
    q, k, v, pos, s, gain = _attn_case(7, m=5, hq=2, hkv=1, d=3)
    tau = 0.8
    got = oracle.gated_attention(q, k, v, pos, s, gain, tau)
    for i in range(5):
        for h in range(2):
            logits = []
            for j in range(5):
                if pos[j] <= pos[i]:
                    dot = sum(q[i, h, c] * k[j, 0, c] for c in range(3))
                    logits.append((j, dot / (math.sqrt(3) * tau) + gain[h] * s[j]))
            top = max(val for _, val in logits)
            w = [(j, math.exp(val - top)) for j, val in logits]
            z = sum(e for _, e in w)
            for c in range(3):
                ref = sum(e * v[j, 0, c] for j, e in w) / z
                assert got[i, h, c] == pytest.approx(ref, abs=1e-13)


def test_attention_invariants():
    q, k, v, pos, s, gain = _attn_case(8)
    tau = 1.1
    base = oracle.gated_attention(q, k, v, pos, s, gain, tau)
    # adding a constant to every kept score only shifts each row's logits
    np.testing.assert_allclose(oracle.gated_attention(q, k, v, pos, s + 3.7, gain, tau), base, atol=1e-12)
    # (Q, tau) == (Q / tau, 1)
    np.testing.assert_allclose(oracle.gated_attention(q / tau, k, v, pos, s, gain, 1.0), base, atol=1e-12)
    # the first kept row sees only itself
    np.testing.assert_allclose(base[0], np.repeat(v[0], 2, axis=0), atol=1e-15)
    # masking on positions equals masking on the row index when positions ascend
    np.testing.assert_allclose(oracle.gated_attention(q, k, v, np.arange(len(pos)), s, gain, tau), base,
                               atol=1e-15)
    # a sampled subset of rows equals the same rows of the full evaluation
    rows = np.array([0, 5, 17, 36])
    np.testing.assert_allclose(oracle.gated_attention(q, k, v, pos, s, gain, tau, rows=rows), base[rows],
                               atol=1e-15)


def test_attention_bias_direction_and_gain_per_query_head():
    q, k, v, pos, s, gain = _attn_case(9, m=12, hq=4, hkv=2, d=8)
    s2 = np.zeros_like(s)
    s2[3] = 60.0                       # one key dominates through its score
    gain2 = np.array([1.0, 0.0, 1.0, 0.0])
    out = oracle.gated_attention(q, k, v, pos, s2, gain2, 1.0)
    for i in range(3, 12):
        np.testing.assert_allclose(out[i, 0], v[3, 0], atol=1e-12)   # head 0 -> kv head 0
        np.testing.assert_allclose(out[i, 2], v[3, 1], atol=1e-12)   # head 2 -> kv head 1
    # gain 0 on heads 1 and 3: identical to the unbiased attention there
    unb = oracle.gated_attention(q, k, v, pos, None, None, 1.0)
    np.testing.assert_allclose(out[:, 1], unb[:, 1], atol=1e-12)
    np.testing.assert_allclose(out[:, 3], unb[:, 3], atol=1e-12)
    # a negative score pushes weight away from its key
    s3 = np.zeros_like(s); s3[0] = -60.0
    out3 = oracle.gated_attention(q, k, v, pos, s3, np.ones(4), 1.0)
    ref = oracle.gated_attention(q[1:], k[1:], v[1:], pos[1:], None, None, 1.0)
    np.testing.assert_allclose(out3[1:], ref, atol=1e-12)


# --------------------------------------------------------------------------- pipeline
def test_full_budget_unbiased_pipeline_equals_causal_attention():
    g = np.random.default_rng(10)
    n, dm, hdim = 40, 12, 6
    x = g.normal(size=(n, dm)); w1 = g.normal(size=(hdim, dm)); w2 = g.normal(size=hdim)
    s = oracle.gate_score(x, w1, None, w2, 0.0)
    kept = oracle.select_topk(s, 0, 32, 32 + 3)
    assert kept.tolist() == list(range(n))
    _, s_kept = oracle.gather_kept(x, s, kept)
    q = g.normal(size=(n, 2, 4)); k = g.normal(size=(n, 1, 4)); v = g.normal(size=(n, 1, 4))
    np.testing.assert_allclose(oracle.gated_attention(q, k, v, kept, s_kept, np.zeros(2), 1.0),
                               oracle.causal_attention(q, k, v), atol=1e-14)


# ---------------------------------------------------------------- several budgets, random-K
def test_splitmix64_known_answers(golden_dir):
    rows = [l for l in open(os.path.join(golden_dir, "splitmix64_seed1234567.txt")) if not l.startswith("#")]
    expect = np.array([int(l) for l in rows], dtype=np.uint64)
    assert np.array_equal(oracle.splitmix64(1234567, len(expect)), expect)
    # the random selector's key of position i is the HIGH half of output i (not the low one)
    assert np.array_equal(oracle.random_keys(1234567, len(expect)), (expect >> np.uint64(32)).astype(np.uint32))


def test_random_keys_are_uniform_and_independent():
    from scipy import stats
    keys = oracle.random_keys(99, 1 << 18)
    # top 6 bits uniform over 64 buckets
    counts = np.bincount(keys >> 26, minlength=64)
    assert stats.chisquare(counts).pvalue > 1e-4
    # every bit is balanced
    bits = (keys[:, None] >> np.arange(32, dtype=np.uint32)) & 1
    assert np.all(np.abs(bits.mean(axis=0) - 0.5) < 0.01)
    # consecutive positions are uncorrelated, and another seed gives another stream
    u = keys.astype(np.float64) / 2.0 ** 32
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 0.01
    assert np.mean(oracle.random_keys(100, 1 << 18) == keys) < 1e-3


def test_select_random_is_a_uniform_subset():
    n, db, de, k = 140, 20, 120, 10
    counts = np.zeros(n)
    for seed in range(600):
        kept = oracle.select_random(n, db, de, k, seed)
        assert len(kept) == (n - (de - db)) + k and np.all(np.diff(kept) > 0)
        assert np.all(np.isin(np.r_[0:db, de:n], kept))
        # the chosen document positions are those holding the k largest keys
        keys = oracle.random_keys(seed, n)
        doc = np.arange(db, de)
        brute = sorted(doc, key=lambda i: (-int(keys[i]), i))[:k]
        assert np.array_equal(np.sort(brute), kept[(kept >= db) & (kept < de)])
        counts[kept] += 1
    # every document position is kept with probability k / D
    from scipy import stats
    doc_counts = counts[db:de]
    assert stats.chisquare(doc_counts).pvalue > 1e-4
    assert abs(doc_counts.mean() / 600 - k / (de - db)) < 1e-12


def test_select_random_edges():
    assert np.array_equal(oracle.select_random(50, 10, 40, 0, 3), np.r_[0:10, 40:50])
    assert np.array_equal(oracle.select_random(50, 10, 40, 99, 3), np.arange(50))
    assert np.array_equal(oracle.select_random(50, 25, 25, 5, 3), np.arange(50))


def test_select_multi_is_each_budget():
    g = np.random.default_rng(4)
    s = np.round(g.normal(size=3000), 1)          # many ties
    ks = [0, 1, 17, 500, 2000, 2999, 5000]
    lists = oracle.select_topk_multi(s, 100, 2900, ks)
    for k, kept in zip(ks, lists):
        doc = np.arange(100, 2900)
        brute = sorted(doc, key=lambda i: (-s[i], i))[:min(k, 2800)]
        assert np.array_equal(kept, np.sort(np.r_[0:100, 2900:3000, brute]))
    for a, b in zip(lists, lists[1:]):
        assert np.all(np.isin(a, b))


# ---------------------------------------------------------------- gradient of the gated attention
def _grad_case(seed, m=9, hq=4, hkv=2, d=8):
    g = np.random.default_rng(seed)
    q, k, v = (g.normal(size=(m, h, d)) for h in (hq, hkv, hkv))
    pos = np.sort(g.choice(3 * m, size=m, replace=False))
    s = g.normal(size=m)
    gain = g.uniform(0.5, 1.5, size=hq)
    dout = g.normal(size=(m, hq, d))
    return q, k, v, pos, s, gain, 1.3, dout


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_backward_matches_torch_autograd(seed):
    q, k, v, pos, s, gain, tau, dout = _grad_case(seed)
    m, hq, d = q.shape
    group = hq // k.shape[1]
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in (("q", q), ("k", k), ("v", v), ("s", s), ("gain", gain), ("tau", np.array(tau)))}
    kk = t["k"].repeat_interleave(group, dim=1)
    vv = t["v"].repeat_interleave(group, dim=1)
    logits = torch.einsum("ihd,jhd->hij", t["q"], kk) / (math.sqrt(d) * t["tau"])
    logits = logits + t["gain"][:, None, None] * t["s"][None, None, :]
    mask = torch.tensor(pos[None, :] <= pos[:, None])
    logits = logits.masked_fill(~mask, float("-inf"))
    out = torch.einsum("hij,jhd->ihd", torch.softmax(logits, dim=-1), vv)
    (out * torch.tensor(dout)).sum().backward()
    dq, dk, dv, ds, dgain, dtau = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, dout)
    for mine, ref in ((dq, t["q"]), (dk, t["k"]), (dv, t["v"]), (ds, t["s"]), (dgain, t["gain"])):
        np.testing.assert_allclose(mine, ref.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert abs(dtau - float(t["tau"].grad)) < 1e-10 * max(1.0, abs(dtau))


def test_attention_backward_matches_finite_differences():
    q, k, v, pos, s, gain, tau, dout = _grad_case(7, m=6, hq=2, hkv=1, d=4)
    grads = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, dout)

    def loss(q_, k_, v_, s_, gain_, tau_):
        return float(np.sum(oracle.gated_attention(q_, k_, v_, pos, s_, gain_, tau_) * dout))

    base = [q, k, v, s, gain, tau]
    eps = 1e-6
    for which, grad in enumerate(grads):
        arr = np.asarray(base[which], dtype=np.float64)
        flat = arr.reshape(-1)
        num = np.zeros(flat.shape)
        for idx in range(flat.size):
            up, dn = flat.copy(), flat.copy()
            up[idx] += eps
            dn[idx] -= eps
            args_u, args_d = list(base), list(base)
            args_u[which] = up.reshape(arr.shape) if arr.ndim else float(up[0])
            args_d[which] = dn.reshape(arr.shape) if arr.ndim else float(dn[0])
            num[idx] = (loss(*args_u) - loss(*args_d)) / (2 * eps)
        np.testing.assert_allclose(np.asarray(grad, dtype=np.float64).reshape(-1), num, rtol=1e-6, atol=1e-8)


def test_attention_lse_and_bias_off_gradients():
    q, k, v, pos, s, gain, tau, dout = _grad_case(3)
    lse = oracle.gated_attention_lse(q, k, v, pos, s, gain, tau)
    # lse of row 0 sees only key 0 (the smallest position)
    d = q.shape[2]
    first = np.argmin(pos)
    for h in range(q.shape[1]):
        z = q[first, h] @ k[first, h // 2] / (math.sqrt(d) * tau) + gain[h] * s[first]
        assert abs(lse[first, h] - z) < 1e-12
    # with the bias off the score gradients are absent and the rest matches gain = 0
    off = oracle.gated_attention_backward(q, k, v, pos, None, None, tau, dout)
    zero = oracle.gated_attention_backward(q, k, v, pos, s, np.zeros_like(gain), tau, dout)
    assert off[3] is None and off[4] is None
    for a, b in zip(off[:3], zero[:3]):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    assert abs(off[5] - zero[5]) < 1e-12


# --------------------------------------------------------------------------- projection, rotary, KV emission
def test_rope_inv_freq_known_values():
    """theta^(-2i/d) at sizes where it is a power of ten, and its constant ratio."""
    np.testing.assert_allclose(oracle.rope_inv_freq(8, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_inv_freq(4, 1e6), [1.0, 1e-3], rtol=1e-15)
    f = oracle.rope_inv_freq(128, 1e6)
    assert f[0] == 1.0 and len(f) == 64
    np.testing.assert_allclose(f[1:] / f[:-1], np.full(63, 1e6 ** (-2.0 / 128)), rtol=1e-13)


def test_rope_is_complex_multiplication():
    """Pairs (i, i + d/2) as complex numbers z_i are multiplied by exp(1j * pos * theta_i)."""
    g = np.random.default_rng(3)
    m, h, d, theta = 40, 3, 16, 5000.0
    x = g.normal(size=(m, h, d))
    pos = g.integers(0, 200000, size=m)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    freq = np.exp(-np.arange(d // 2) * (2.0 / d) * np.log(theta))
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(oracle.rope(x, pos, theta), want, rtol=1e-9, atol=1e-9)


def test_rope_group_and_relative_position_properties():
    g = np.random.default_rng(4)
    m, d, theta = 30, 32, 1e6
    x = g.normal(size=(m, 2, d))
    p1 = g.integers(0, 5000, size=m)
    p2 = g.integers(0, 5000, size=m)
    # identity at position 0, composition adds positions, each pair keeps its length
    np.testing.assert_array_equal(oracle.rope(x, np.zeros(m), theta), x)
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, p1, theta), p2, theta), oracle.rope(x, p1 + p2, theta),
                               atol=1e-9)
    r = oracle.rope(x, p1, theta)
    np.testing.assert_allclose(r[..., :d // 2] ** 2 + r[..., d // 2:] ** 2, x[..., :d // 2] ** 2 + x[..., d // 2:] ** 2,
                               rtol=1e-12)
    # the rotated q.k depends on the positions only through their difference
    q, k = x[:, 0:1, :], x[:, 1:2, :]
    shift = 777
    a = np.sum(oracle.rope(q, p1, theta) * oracle.rope(k, p2, theta), axis=-1)
    b = np.sum(oracle.rope(q, p1 + shift, theta) * oracle.rope(k, p2 + shift, theta), axis=-1)
    np.testing.assert_allclose(a, b, atol=1e-9)
    # swapping the halves' roles (a transposed pairing) breaks the property above
    bad = np.concatenate([x[..., d // 2:], x[..., :d // 2]], axis=-1)
    assert not np.allclose(oracle.rope(bad, p1, theta), oracle.rope(x, p1, theta))


def test_qkv_projection_matches_torch_linear():
    """At position 0 the rotation is the identity: q, k, v are slices of a torch Linear."""
    g = np.random.default_rng(5)
    m, d_model, hq, hkv, d = 20, 48, 4, 2, 8
    x = g.normal(size=(m, d_model))
    w = g.normal(size=((hq + 2 * hkv) * d, d_model))
    b = g.normal(size=(hq + 2 * hkv) * d)
    lin = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    q, k, v = oracle.qkv_rope(x, w, b, hq, hkv, d, np.zeros(m), 1e4)
    np.testing.assert_allclose(q.reshape(m, -1), lin[:, : hq * d], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k.reshape(m, -1), lin[:, hq * d:(hq + hkv) * d], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v.reshape(m, -1), lin[:, (hq + hkv) * d:], rtol=1e-12, atol=1e-12)
    # at other positions q and k are rotated, v is not
    pos = g.integers(0, 100000, size=m)
    q2, k2, v2 = oracle.qkv_rope(x, w, None, hq, hkv, d, pos, 1e4)
    q0, k0, v0 = oracle.qkv_rope(x, w, None, hq, hkv, d, np.zeros(m), 1e4)
    np.testing.assert_allclose(q2, oracle.rope(q0, pos, 1e4), atol=1e-10)
    np.testing.assert_allclose(k2, oracle.rope(k0, pos, 1e4), atol=1e-10)
    np.testing.assert_array_equal(v2, v0)


def test_emit_kv_writes_only_its_slots():
    g = np.random.default_rng(6)
    cap, hkv, d, m, slot0 = 50, 2, 4, 7, 20
    kc, vc, pc = g.normal(size=(cap, hkv, d)), g.normal(size=(cap, hkv, d)), g.integers(0, 9, size=cap)
    k, v, pos = g.normal(size=(m, hkv, d)), g.normal(size=(m, hkv, d)), np.arange(m) * 3
    kc2, vc2, pc2 = oracle.emit_kv(kc, vc, pc, slot0, k, v, pos)
    keep = np.r_[0:slot0, slot0 + m:cap]
    np.testing.assert_array_equal(kc2[keep], kc[keep])
    np.testing.assert_array_equal(vc2[keep], vc[keep])
    np.testing.assert_array_equal(pc2[keep], pc[keep])
    np.testing.assert_array_equal(kc2[slot0:slot0 + m], k)
    np.testing.assert_array_equal(vc2[slot0:slot0 + m], v)
    np.testing.assert_array_equal(pc2[slot0:slot0 + m], pos)


@pytest.mark.parametrize("bias", [True, False])
def test_backward_rows_equal_the_whole_gradient(bias):
    """The per-row form (P from the forward's lse, D_i = dout_i . out_i) gives the same rows as
    the whole-matrix gradient, which autograd and finite differences pin above."""
    g = np.random.default_rng(21 + bias)
    m, hq, hkv, d = 70, 4, 2, 16
    q, k, v, dout = (g.normal(size=(m, h, d)) for h in (hq, hkv, hkv, hq))
    pos = np.sort(g.choice(300, m, replace=False))
    s = g.normal(size=m) * 2 if bias else None
    gain = g.uniform(0.5, 1.5, size=hq) if bias else None
    tau = 0.9
    out = oracle.gated_attention(q, k, v, pos, s, gain, tau)
    lse = oracle.gated_attention_lse(q, k, v, pos, s, gain, tau)
    dq, dk, dv, ds, _, _ = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, dout)
    qr, kr = np.array([0, 5, 33, m - 1]), np.array([0, 17, 40, m - 1])
    rq, rk, rv, rs = oracle.gated_attention_backward_rows(q, k, v, pos, s, gain, tau, dout, out, lse, qr, kr)
    assert np.allclose(rq, dq[qr], rtol=1e-10, atol=1e-12)
    assert np.allclose(rk, dk[kr], rtol=1e-10, atol=1e-12)
    assert np.allclose(rv, dv[kr], rtol=1e-10, atol=1e-12)
    if bias:
        assert np.allclose(rs, ds[kr], rtol=1e-10, atol=1e-12)
    else:
        assert rs is None
    # the row subset of the log-sum-exp is the same rows of the whole one
    assert np.allclose(oracle.gated_attention_lse(q, k, v, pos, s, gain, tau, rows=qr), lse[qr], rtol=0, atol=1e-13)


def test_backward_magnitudes_bound_the_gradients():
    """The per-element sums of absolute terms (the tolerance scale of the GPU gradient tests)
    bound every gradient element; with dout >= 0 every term of dv is non-negative, so dv's
    magnitude IS dv; flipping dout's sign flips the gradients and leaves the magnitudes; the
    per-row form gives the same magnitudes as the whole-matrix form."""
    g = np.random.default_rng(31)
    m, hq, hkv, d = 60, 4, 2, 16
    q, k, v, dout = (g.normal(size=(m, h, d)) for h in (hq, hkv, hkv, hq))
    pos = np.sort(g.choice(200, m, replace=False))
    s = g.normal(size=m) * 2
    gain = g.uniform(0.5, 1.5, size=hq)
    tau = 1.1
    res = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, dout, magnitudes=True)
    dq, dk, dv, ds, dgain, dtau, mag = res
    for name, gr in (("dq", dq), ("dk", dk), ("dv", dv), ("ds_kept", ds)):
        assert np.all(np.abs(gr) <= mag[name] * (1 + 1e-12) + 1e-15), name
        assert np.all(mag[name] >= 0)
    assert np.all(np.abs(dgain) <= mag["dgain"] * (1 + 1e-12))
    assert abs(dtau) <= mag["dtau"] * (1 + 1e-12)
    # dout >= 0: dv's terms P_ij dout_i are all non-negative
    dpos = np.abs(dout)
    _, _, dv2, _, _, _, mag2 = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, dpos, magnitudes=True)
    np.testing.assert_allclose(mag2["dv"], dv2, rtol=1e-12, atol=1e-14)
    # sign of dout
    neg = oracle.gated_attention_backward(q, k, v, pos, s, gain, tau, -dout, magnitudes=True)
    for a, b in zip(neg[:4], res[:4]):
        np.testing.assert_allclose(a, -b, rtol=1e-12, atol=1e-14)
    for name in ("dq", "dk", "dv", "ds_kept"):
        np.testing.assert_allclose(neg[6][name], mag[name], rtol=1e-12, atol=1e-14)
    # rows form
    out = oracle.gated_attention(q, k, v, pos, s, gain, tau)
    lse = oracle.gated_attention_lse(q, k, v, pos, s, gain, tau)
    qr, kr = np.array([0, 9, 31, m - 1]), np.array([0, 12, 44, m - 1])
    *_, rmag = oracle.gated_attention_backward_rows(q, k, v, pos, s, gain, tau, dout, out, lse, qr, kr,
                                                    magnitudes=True)
    np.testing.assert_allclose(rmag["dq"], mag["dq"][qr], rtol=1e-10)
    np.testing.assert_allclose(rmag["dk"], mag["dk"][kr], rtol=1e-10)
    np.testing.assert_allclose(rmag["dv"], mag["dv"][kr], rtol=1e-10)
    np.testing.assert_allclose(rmag["ds_kept"], mag["ds_kept"][kr], rtol=1e-10)
    for name in ("dq", "dk", "dv", "ds_kept"):
        sub = qr if name == "dq" else kr
        np.testing.assert_allclose(rmag[name + "_rss"], mag[name + "_rss"][sub], rtol=1e-10)
    # root-sum-square <= sum of absolute values, element by element
    for name in ("dq", "dk", "dv", "ds_kept"):
        assert np.all(mag[name + "_rss"] <= mag[name] * (1 + 1e-12) + 1e-15), name
    # a single query and key: P = 1 and every gradient element is one term per head, so
    # dv's root-sum-square over the group's query heads is the norm of their dout values
    one = oracle.gated_attention_backward(q[:1], k[:1], v[:1], pos[:1], s[:1], gain, tau, dout[:1],
                                          magnitudes=True)[6]
    grp = hq // hkv
    np.testing.assert_allclose(one["dv_rss"][0], np.sqrt((dout[0] ** 2).reshape(hkv, grp, d).sum(axis=1)),
                               rtol=1e-12)
