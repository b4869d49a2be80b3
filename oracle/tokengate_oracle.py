"""Float64 CPU oracle for TokenGate's gated-prefill path.

TEST INFRASTRUCTURE ONLY.  This module is the independent checker of the HIP
path: only the test-suite, the smoke check and the benchmark's CPU-baseline leg
may import or run it.  It shares no code with the HIP library and imports
nothing from the product package.  Every function is a plain, slow, literal
statement of what the TokenGate pages define, in float64 NumPy.

Sources (pages are cited by site and title; sections by their headings):
  [P1] aiproducthub.cn, "斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情
  [P2] aisight.pl, "TokenGate: Stanford i Berkeley ucza model, ktore tokeny
       pominac przy czytaniu dlugiego kontekstu", section "Jak to dziala"
  [P4] news.chathome.org TokenGate article, sections
       "TokenGate の学習可能なトークンプルーニングの仕組み" and
       "トークンゲート付きアテンションとは"

The pages give the method in words only.  The formula of the gated attention
logit, q.k / (sqrt(d) tau) + g_h s_j under a causal mask on original positions,
is the specification adopted here for those words.  Readings taken where
the pages are silent are listed with each function.

Parity status: every function here is pinned by CPU tests against library
routines (torch's GELU / normal CDF, Linear layers and scaled_dot_product_attention
in float64), brute-force sorting, tabulated normal-CDF values and invariants.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "gelu", "gate_score", "num_kept", "select_topk", "select_topk_multi", "splitmix64", "random_keys",
    "select_random", "gather_kept", "gated_attention", "causal_attention", "gated_attention_lse",
    "gated_attention_backward", "gated_attention_backward_rows", "rope_inv_freq", "rope", "qkv_rope", "emit_kv",
]


# ----------------------------------------------------------------------------------------
# (1) gate scorer  [P1 事件详情; P2 "Jak to dziala"; P4 仕組み]
# A small MLP maps each token's post-attention residual at the gate layer to one
# scalar score.  Form d_model -> d_hidden -> 1 with a GELU between the layers.
# Reading: "GELU" is the exact one, x * Phi(x) with Phi the standard normal CDF
# (not the tanh approximation).  b1 and b2 are optional (zero in the workloads).
# ----------------------------------------------------------------------------------------
def gelu(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def gate_score(x, w1, b1, w2, b2=0.0):
    """s[i] = b2 + sum_j w2[j] * GELU(b1[j] + sum_k x[i,k] * w1[j,k]).

    x: [N, d_model]; w1: [d_hidden, d_model] (output-by-input layout);
    b1: [d_hidden] or None; w2: [d_hidden]; b2: scalar.  Returns float64 [N].
    """
    x = np.asarray(x, dtype=np.float64)
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    h = x @ w1.T
    if b1 is not None:
        h = h + np.asarray(b1, dtype=np.float64)[None, :]
    a = gelu(h)
    return a @ w2 + float(b2)


# ----------------------------------------------------------------------------------------
# (2) top-K selection over the document only  [P1 事件详情; P2 "Jak to dziala"; P4 仕組み]
# Only the document part of the prompt can be pruned; the question is always kept.
# Of the document tokens, the K highest-scoring ones are kept.  Kept tokens are
# listed in ascending original position ("stable position order").
# Readings: K counts document tokens only and is clamped to D = doc_end - doc_begin;
# ties go to the lower position; -0 equals +0; NaN ranks below every number
# (including -inf), ties among NaNs again to the lower position.
# ----------------------------------------------------------------------------------------
def num_kept(n, doc_begin, doc_end, k):
    d = doc_end - doc_begin
    return (n - d) + min(k, d)


def select_topk(scores, doc_begin, doc_end, k):
    """Kept positions (int64, ascending): every non-document position plus the
    min(k, D) best document positions, found through the K-th largest value."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if not (0 <= doc_begin <= doc_end <= n) or k < 0:
        raise ValueError("bad selection arguments")
    d = doc_end - doc_begin
    k_eff = min(k, d)
    pos = np.arange(doc_begin, doc_end, dtype=np.int64)
    vals = s[doc_begin:doc_end]
    is_nan = np.isnan(vals)
    num_pos, num_vals = pos[~is_nan], vals[~is_nan]
    nan_pos = pos[is_nan]

    if k_eff <= len(num_vals):
        if k_eff == 0:
            chosen = np.zeros(0, dtype=np.int64)
        else:
            # threshold t = the k_eff-th largest number; keep everything above it,
            # then fill the remaining quota from the values equal to t, lowest
            # positions first.
            t = np.partition(num_vals, len(num_vals) - k_eff)[len(num_vals) - k_eff]
            above = num_pos[num_vals > t]
            need = k_eff - len(above)
            at_t = num_pos[num_vals == t]          # already ascending
            chosen = np.concatenate([above, at_t[:need]])
    else:
        # every number is kept; NaNs fill the rest, lowest positions first
        chosen = np.concatenate([num_pos, nan_pos[:k_eff - len(num_vals)]])

    outside = np.concatenate([np.arange(0, doc_begin, dtype=np.int64),
                              np.arange(doc_end, n, dtype=np.int64)])
    return np.sort(np.concatenate([outside, chosen]).astype(np.int64))


# ----------------------------------------------------------------------------------------
# (2b) several budgets over the same scores  [P1 事件详情; P2 "Wyniki"]
# One trained gate serves every budget, so the same scores are selected at several
# budgets: each budget's kept list is the single-budget selection at that budget.
# ----------------------------------------------------------------------------------------
def select_topk_multi(scores, doc_begin, doc_end, ks):
    """[select_topk(scores, doc_begin, doc_end, k) for k in ks]."""
    return [select_topk(scores, doc_begin, doc_end, k) for k in ks]


# ----------------------------------------------------------------------------------------
# (2c) random-K selector  [P1 事件详情; P4 "ベンチマーク"]
# The pages' ablation keeps a random set of K document tokens (question kept) on the
# same backbone.  Reading: a uniformly random min(k, D)-subset of the document, drawn
# reproducibly from a seed -- every position gets an independent uniform 32-bit key and
# the K largest keys are kept (equal keys: lower position first, as for scores).
# Keys: SplitMix64 (Steele, Lea, Flood, "Fast Splittable Pseudorandom Number
# Generators", OOPSLA 2014), the key of position i being the high 32 bits of the i-th
# output (i = 0, 1, ...) of the generator seeded with `seed`: the state advances by the
# golden-ratio increment 0x9E3779B97F4A7C15 before each output, and the output is the
# state passed through the variant-13 finaliser (xor-shift 30, multiply
# 0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).
# ----------------------------------------------------------------------------------------
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed, count):
    """The first `count` outputs of SplitMix64 seeded with `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + _GOLDEN * np.arange(1, count + 1, dtype=np.uint64)
        z = state
        z = (z ^ (z >> np.uint64(30))) * _MIX1
        z = (z ^ (z >> np.uint64(27))) * _MIX2
        return z ^ (z >> np.uint64(31))


def random_keys(seed, n):
    """Key of positions 0..n-1: high 32 bits of the SplitMix64 outputs (uint32)."""
    return (splitmix64(seed, n) >> np.uint64(32)).astype(np.uint32)


def select_random(n, doc_begin, doc_end, k, seed):
    """Kept positions of the random-K selector (int64, ascending)."""
    keys = random_keys(seed, n).astype(np.float64)    # exact: keys < 2^32
    return select_topk(keys, doc_begin, doc_end, k)


# ----------------------------------------------------------------------------------------
# (3) gather  [P1 事件详情; P2 "Jak to dziala"; P4 仕組み]
# Layers above the gate process only the kept tokens; pruned tokens create no
# KV entries.  The kept rows (and their scores) are compacted in position order.
# ----------------------------------------------------------------------------------------
def gather_kept(x, scores, kept):
    kept = np.asarray(kept, dtype=np.int64)
    return np.asarray(x)[kept], np.asarray(scores)[kept]


# ----------------------------------------------------------------------------------------
# (4) token-gated attention  [P1 事件详情; P2 "Jak to dziala"; P4 トークンゲート付きアテンションとは]
# Each kept key's score becomes a bias on the attention logits above the gate,
# scaled by a learnable per-head gain; a learnable temperature corrects for each
# query seeing fewer keys.  Adopted form:
#     logit[i, j] = q_i . k_j / (sqrt(d) * tau) + gain[h] * s_kept[j],   pos_j <= pos_i
# Readings: tau scales the q.k term only; gain is per query head; grouped-query
# heads share key/value head g(h) = h // (Hq / Hkv); question tokens carry their
# own score as bias like every kept key; s_kept=None or gain=None turns the bias off.
# ----------------------------------------------------------------------------------------
def gated_attention(q, k, v, pos, s_kept, gain, tau, rows=None, block=512):
    """q: [M, Hq, d]; k, v: [M, Hkv, d]; pos: [M] original positions.
    Returns float64 [len(rows), Hq, d] (all rows when rows is None)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    m, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    use_bias = s_kept is not None and gain is not None
    if use_bias:
        s_kept = np.asarray(s_kept, dtype=np.float64)
        gain = np.asarray(gain, dtype=np.float64)
    scale = 1.0 / (math.sqrt(d) * float(tau))
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    for r0 in range(0, len(rows), block):
        rb = rows[r0:r0 + block]
        visible = pos[None, :] <= pos[rb][:, None]          # [b, M]
        for h in range(hq):
            g = h // group
            logits = (q[rb, h, :] @ k[:, g, :].T) * scale
            if use_bias:
                logits = logits + gain[h] * s_kept[None, :]
            logits = np.where(visible, logits, -np.inf)
            mx = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - mx)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + len(rb), h, :] = p @ v[:, g, :]
    return out


def causal_attention(q, k, v, rows=None):
    """Ordinary causal grouped-query attention: the gated form with the bias off,
    tau = 1 and positions 0..M-1."""
    m = np.asarray(q).shape[0]
    return gated_attention(q, k, v, np.arange(m), None, None, 1.0, rows=rows)


# ----------------------------------------------------------------------------------------
# (5) gradient of the token-gated attention  [P1 事件详情; P2 "Jak to dziala";
#     P4 トークンゲート付きアテンションとは]
# Top-K is not differentiable; the score enters the attention logits as a bias
# precisely so that the loss has a gradient path back into the scorer (and into the
# per-head gain and the temperature).  For a loss L with dL/dout = dout, by the chain
# rule through softmax (P = softmax of the visible logits per row):
#     dP[i, j]   = dout_i . v_j
#     D_i        = sum_j P[i, j] dP[i, j]        (= dout_i . out_i)
#     dZ[i, j]   = P[i, j] (dP[i, j] - D_i)      (gradient of the logit)
#     dq_i       = sum_j dZ[i, j] k_j / (sqrt(d) tau)
#     dk_j      += sum_i dZ[i, j] q_i / (sqrt(d) tau)      (summed over the heads of the group)
#     dv_j      += sum_i P[i, j] dout_i                    (summed over the heads of the group)
#     ds_kept_j  = sum_h gain[h] sum_i dZ_h[i, j]
#     dgain[h]   = sum_j s_kept[j] sum_i dZ_h[i, j]
#     dtau       = -(1 / tau) sum_{h,i,j} dZ_h[i, j] q_i . k_j / (sqrt(d) tau)
# ----------------------------------------------------------------------------------------
def gated_attention_lse(q, k, v, pos, s_kept, gain, tau, rows=None):
    """Natural-log log-sum-exp of each row's visible logits: float64 [len(rows), Hq]
    (all M rows when rows is None)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    m, hq, d = q.shape
    rows = np.arange(m, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    group = hq // k.shape[1]
    use_bias = s_kept is not None and gain is not None
    scale = 1.0 / (math.sqrt(d) * float(tau))
    visible = pos[None, :] <= pos[rows][:, None]
    lse = np.empty((len(rows), hq))
    for h in range(hq):
        logits = (q[rows, h, :] @ k[:, h // group, :].T) * scale
        if use_bias:
            logits = logits + float(gain[h]) * np.asarray(s_kept, dtype=np.float64)[None, :]
        logits = np.where(visible, logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        lse[:, h] = (mx + np.log(np.exp(logits - mx).sum(axis=1, keepdims=True)))[:, 0]
    return lse


def gated_attention_backward(q, k, v, pos, s_kept, gain, tau, dout, magnitudes=False):
    """Gradients (dq, dk, dv, ds_kept, dgain, dtau) of sum(out * dout), float64.
    ds_kept and dgain are None when the bias is off.

    With magnitudes=True a seventh item is returned: a dict holding, for every output,
    the same expression with every sum taken over the absolute values of its terms --
    the scale against which a rounding error in that output is judged (the outputs are
    sums whose terms cancel: each row of dZ sums to zero, and dZ itself is a difference):
        |dP|_ij   = |dout_i| . |v_j|,   |D|_i = |dout_i| . |out_i|   (D_i = dout_i . out_i)
        |dZ|_ij   = P_ij (|dP|_ij + |D|_i)
        "dq"      [M, Hq, d]  scale sum_j |dZ|_ij |k_j|
        "dk"      [M, Hkv, d] scale sum_{h in g} sum_i |dZ|_ij |q_i|
        "dv"      [M, Hkv, d] sum_{h in g} sum_i P_ij |dout_i|
        "ds_kept" [M]         sum_h |gain_h| sum_i |dZ|_ij          (None when the bias is off)
        "dgain"   [Hq]        sum_j |s_j| |sum_i dZ_ij|
        "dtau"    float       sum |dZ_ij q_i.k_j| scale / tau
    and, for dq, dk, dv and ds_kept, the root-sum-square of the same terms ("dq_rss", ...),
    the size that independent rounding errors of the terms add up to, with the term of dZ
    taken as a_ij = P_ij (|dout_i . v_j| + |D_i|):
        "dq_rss" = scale sqrt(sum_j a_ij^2 k_j^2)        "dk_rss" = scale sqrt(sum_{h,i} a_ij^2 q_i^2)
        "dv_rss" = sqrt(sum_{h,i} P_ij^2 dout_i^2)       "ds_kept_rss" = sqrt(sum_h gain_h^2 sum_i a_ij^2)"""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    m, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    use_bias = s_kept is not None and gain is not None
    if use_bias:
        s_kept = np.asarray(s_kept, dtype=np.float64)
        gain = np.asarray(gain, dtype=np.float64)
    scale = 1.0 / (math.sqrt(d) * float(tau))
    visible = pos[None, :] <= pos[:, None]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    ds = np.zeros(m) if use_bias else None
    dgain = np.zeros(hq) if use_bias else None
    dtau = 0.0
    mag_gain = np.zeros(hq)
    mag_tau = 0.0
    if magnitudes:
        mag_dq, mag_dk, mag_dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        mag_ds = np.zeros(m) if use_bias else None
        sq_dq, sq_dk, sq_dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)   # sums of squares
        sq_ds = np.zeros(m) if use_bias else None
    for h in range(hq):
        g = h // group
        qk = q[:, h, :] @ k[:, g, :].T
        logits = qk * scale
        if use_bias:
            logits = logits + gain[h] * s_kept[None, :]
        logits = np.where(visible, logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - mx)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[:, g, :]
        dp = dout[:, h, :] @ v[:, g, :].T
        dsum = np.sum(dout[:, h, :] * o, axis=1, keepdims=True)
        dz = p * (dp - dsum)
        dq[:, h, :] = (dz @ k[:, g, :]) * scale
        dk[:, g, :] += (dz.T @ q[:, h, :]) * scale
        dv[:, g, :] += p.T @ dout[:, h, :]
        if use_bias:
            col = dz.sum(axis=0)
            ds += gain[h] * col
            dgain[h] = float(np.dot(col, s_kept))
            mag_gain[h] = float(np.dot(np.abs(col), np.abs(s_kept)))
        dtau += -float(np.sum(dz * qk)) * scale / float(tau)
        mag_tau += float(np.sum(np.abs(dz * qk))) * scale / float(tau)
        if magnitudes:
            adz = p * (np.abs(dout[:, h, :]) @ np.abs(v[:, g, :]).T
                       + np.sum(np.abs(dout[:, h, :] * o), axis=1, keepdims=True))
            mag_dq[:, h, :] = (adz @ np.abs(k[:, g, :])) * scale
            mag_dk[:, g, :] += (adz.T @ np.abs(q[:, h, :])) * scale
            mag_dv[:, g, :] += p.T @ np.abs(dout[:, h, :])
            if use_bias:
                mag_ds += abs(gain[h]) * adz.sum(axis=0)
            a2 = (p * (np.abs(dp) + np.abs(dsum))) ** 2
            sq_dq[:, h, :] = (a2 @ k[:, g, :] ** 2) * scale ** 2
            sq_dk[:, g, :] += (a2.T @ q[:, h, :] ** 2) * scale ** 2
            sq_dv[:, g, :] += (p ** 2).T @ dout[:, h, :] ** 2
            if use_bias:
                sq_ds += gain[h] ** 2 * a2.sum(axis=0)
    if magnitudes:
        return dq, dk, dv, ds, dgain, dtau, {"dq": mag_dq, "dk": mag_dk, "dv": mag_dv, "ds_kept": mag_ds,
                                             "dgain": mag_gain, "dtau": mag_tau,
                                             "dq_rss": np.sqrt(sq_dq), "dk_rss": np.sqrt(sq_dk),
                                             "dv_rss": np.sqrt(sq_dv),
                                             "ds_kept_rss": np.sqrt(sq_ds) if use_bias else None}
    return dq, dk, dv, ds, dgain, dtau


def gated_attention_backward_rows(q, k, v, pos, s_kept, gain, tau, dout, out, lse, q_rows, k_rows,
                                  magnitudes=False):
    """Selected rows of the same gradient, float64: dq at the query rows q_rows, and dk, dv
    and ds_kept at the key rows k_rows (ds_kept None when the bias is off), given the
    forward's output `out` [M, Hq, d] and natural-log log-sum-exp `lse` [M, Hq].

    With those two, every term is local to one row or one key: the softmax weight of key j
    for query i is P_ij = exp(z_ij - lse_i) (z the gated logit, -inf where pos_j > pos_i),
    the row's correction is D_i = dout_i . out_i (= sum_j P_ij dout_i . v_j), and the logit
    gradient is dZ_ij = P_ij (dout_i . v_j - D_i).  Then dq_i = scale sum_j dZ_ij k_j,
    dk_j = scale sum_i dZ_ij q_i and dv_j = sum_i P_ij dout_i (summed over the query heads
    of the key's group), ds_j = sum_h gain_h sum_i dZ_ij.  A row costs O(M d) per head,
    so sampled rows of a large problem are cheap where the whole gradient is not.

    With magnitudes=True a fifth item is returned: the per-element sums of absolute terms
    and root-sum-squares of the terms of dq, dk, dv and ds_kept at those rows, as
    gated_attention_backward defines them."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    m, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    use_bias = s_kept is not None and gain is not None
    if use_bias:
        s_kept = np.asarray(s_kept, dtype=np.float64)
        gain = np.asarray(gain, dtype=np.float64)
    scale = 1.0 / (math.sqrt(d) * float(tau))
    dsum = np.sum(dout * out, axis=2)                          # D_i per head: [M, Hq]
    dsum_abs = np.sum(np.abs(dout * out), axis=2)              # its terms' magnitudes
    # per-head [M, d] slices, contiguous (each is read once per selected row)
    qh = [np.ascontiguousarray(q[:, h, :]) for h in range(hq)]
    doh = [np.ascontiguousarray(dout[:, h, :]) for h in range(hq)]
    kg = [np.ascontiguousarray(k[:, g, :]) for g in range(hkv)]
    vg = [np.ascontiguousarray(v[:, g, :]) for g in range(hkv)]
    dq = np.zeros((len(q_rows), hq, d))
    mq, sqq = np.zeros_like(dq), np.zeros_like(dq)
    for a, i in enumerate(q_rows):
        visible = pos <= pos[i]
        for h in range(hq):
            g = h // group
            z = (kg[g] @ q[i, h, :]) * scale
            if use_bias:
                z = z + gain[h] * s_kept
            p = np.where(visible, np.exp(np.where(visible, z, 0.0) - lse[i, h]), 0.0)
            dp = vg[g] @ dout[i, h, :]
            dz = p * (dp - dsum[i, h])
            dq[a, h, :] = scale * (dz @ kg[g])
            if magnitudes:
                adz = p * (np.abs(vg[g]) @ np.abs(dout[i, h, :]) + dsum_abs[i, h])
                mq[a, h, :] = scale * (adz @ np.abs(kg[g]))
                sqq[a, h, :] = scale ** 2 * ((p * (np.abs(dp) + abs(dsum[i, h]))) ** 2 @ kg[g] ** 2)
    dk = np.zeros((len(k_rows), hkv, d))
    dv = np.zeros((len(k_rows), hkv, d))
    ds = np.zeros(len(k_rows)) if use_bias else None
    mk, mv = np.zeros_like(dk), np.zeros_like(dv)
    ms = np.zeros(len(k_rows)) if use_bias else None
    sqk, sqv = np.zeros_like(dk), np.zeros_like(dv)
    sqs = np.zeros(len(k_rows)) if use_bias else None
    for b, j in enumerate(k_rows):
        visible = pos[j] <= pos                                 # query rows that see key j
        for h in range(hq):
            g = h // group
            z = (qh[h] @ k[j, g, :]) * scale
            if use_bias:
                z = z + gain[h] * s_kept[j]
            p = np.where(visible, np.exp(np.where(visible, z, 0.0) - lse[:, h]), 0.0)
            dp = doh[h] @ v[j, g, :]
            dz = p * (dp - dsum[:, h])
            dk[b, g, :] += scale * (dz @ qh[h])
            dv[b, g, :] += p @ doh[h]
            if use_bias:
                ds[b] += gain[h] * dz.sum()
            if magnitudes:
                adz = p * (np.abs(doh[h]) @ np.abs(v[j, g, :]) + dsum_abs[:, h])
                mk[b, g, :] += scale * (adz @ np.abs(qh[h]))
                mv[b, g, :] += p @ np.abs(doh[h])
                if use_bias:
                    ms[b] += abs(gain[h]) * adz.sum()
                a2 = (p * (np.abs(dp) + np.abs(dsum[:, h]))) ** 2
                sqk[b, g, :] += scale ** 2 * (a2 @ qh[h] ** 2)
                sqv[b, g, :] += p ** 2 @ doh[h] ** 2
                if use_bias:
                    sqs[b] += gain[h] ** 2 * a2.sum()
    if magnitudes:
        return dq, dk, dv, ds, {"dq": mq, "dk": mk, "dv": mv, "ds_kept": ms, "dq_rss": np.sqrt(sqq),
                                "dk_rss": np.sqrt(sqk), "dv_rss": np.sqrt(sqv),
                                "ds_kept_rss": np.sqrt(sqs) if use_bias else None}
    return dq, dk, dv, ds


# ----------------------------------------------------------------------------------------
# (6) kept-row projection and KV emission  [P1 事件详情; P2 "Jak to dziala"; P4 仕組み]
# Layers above the gate run on the kept tokens only, and pruned tokens get no KV
# entries.  The step after the gather: project the kept hidden states to Q, K, V,
# rotate Q and K by their ORIGINAL positions, and write K, V (and the positions)
# into a cache that holds the kept tokens only, compacted.
# Readings (the pages are silent on all of these): one fused weight W_qkv
# [(Hq + 2 Hkv) d, d_model] (rows: the Hq query heads, then the Hkv key heads, then
# the Hkv value heads; optional bias); rotary embedding in the rotate-half form,
# feature i paired with i + d/2 and turned by the angle pos * theta^(-2 i / d); no
# per-head normalisation before the rotation.
# ----------------------------------------------------------------------------------------
def rope_inv_freq(head_dim, theta):
    """theta^(-2 i / d) for i = 0 .. d/2 - 1, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope(x, pos, theta):
    """Rotate-half rotary embedding of x [M, H, d] at positions pos [M], float64:
    out[:, :, i] = x_i cos a - x_{i+d/2} sin a,  out[:, :, i+d/2] = x_{i+d/2} cos a + x_i sin a,
    a = pos * theta^(-2 i / d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]   # [M, d/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    lo, hi = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def qkv_rope(x_kept, w_qkv, b_qkv, n_q_heads, n_kv_heads, head_dim, pos, theta):
    """(q [M, Hq, d], k [M, Hkv, d], v [M, Hkv, d]) float64 from the kept rows
    x_kept [M, d_model]: C = x_kept W_qkv^T (+ b_qkv), split by heads, rotary on q and k."""
    x = np.asarray(x_kept, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    c = x @ w.T
    if b_qkv is not None:
        c = c + np.asarray(b_qkv, dtype=np.float64)[None, :]
    m = x.shape[0]
    nq, nk = n_q_heads * head_dim, n_kv_heads * head_dim
    q = c[:, :nq].reshape(m, n_q_heads, head_dim)
    k = c[:, nq:nq + nk].reshape(m, n_kv_heads, head_dim)
    v = c[:, nq + nk:nq + 2 * nk].reshape(m, n_kv_heads, head_dim)
    return rope(q, pos, theta), rope(k, pos, theta), v


def emit_kv(k_cache, v_cache, pos_cache, slot0, k, v, pos):
    """Copies of the caches with rows slot0 .. slot0 + M - 1 holding the kept tokens'
    k, v and positions; every other row unchanged (pos_cache may be None)."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    m = len(k)
    kc[slot0:slot0 + m] = k
    vc[slot0:slot0 + m] = v
    pc = None
    if pos_cache is not None:
        pc = np.array(pos_cache, copy=True)
        pc[slot0:slot0 + m] = pos
    return kc, vc, pc
