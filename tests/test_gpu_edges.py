"""GPU edge cases of each entry point against the float64 oracle: ragged sizes,
tie-adversarial and non-finite scores, empty / full / middle document spans,
every supported head grouping and head_dim, bias off, gapped positions, strided
and unaligned inputs, and workspace reuse across calls of different sizes."""
import numpy as np
import pytest

import oracle
from learned_token_pruning_scorer_amd import inputs
from gpu_common import ATTN_MAX_TOL, ATTN_MEAN_TOL, SCORE_TOL, host_f64, log, require_gpu

pytestmark = pytest.mark.gpu


# --------------------------------------------------------------------------- selection
def _select_cases():
    g = np.random.default_rng(7)
    cases = []
    cases.append(("n1", np.array([0.5]), 0, 1, [0, 1, 5]))
    cases.append(("all-equal", np.full(1000, 0.25), 100, 900, [1, 399, 800, 900]))
    cases.append(("int-ties", g.integers(-3, 4, size=5000).astype(np.float64), 0, 4990, [1, 17, 2500, 4989]))
    pool = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, 2.5])
    cases.append(("nonfinite", pool[g.integers(0, len(pool), size=3000)], 10, 2990, [0, 1, 500, 1500, 2979, 2980]))
    cases.append(("doc-middle", g.normal(size=4096), 1000, 2000, [0, 1, 100, 999, 1000, 5000]))
    cases.append(("empty-doc", g.normal(size=2048), 500, 500, [0, 3]))
    cases.append(("ragged-1025", g.normal(size=1025), 0, 1000, [1, 500, 999]))
    cases.append(("ragged-2047", g.normal(size=2047), 47, 2047, [1, 1000, 1999]))
    # keys that share their top 24 bits: exercises the last digit pass
    near = (1.0 + np.arange(3000) % 50 * np.finfo(np.float32).eps).astype(np.float32).astype(np.float64)
    cases.append(("low-bits", g.permutation(near), 0, 3000, [1, 61, 1500, 2999]))
    big = np.round(g.normal(size=300000) * 64) / 64
    cases.append(("large-ties", big, 0, 299000, [12345, 150000]))
    cases.append(("all-equal-large", np.full(140000, 0.25), 0, 139000, [1, 70000, 138999]))
    cases.append(("coarse-ties-large", np.round(g.normal(size=131072) * 4) / 4, 0, 131008, [8192, 60000]))
    cases.append(("normal-131072", g.normal(size=131072), 0, 131008, [1, 8192, 131007]))
    cases.append(("ties-32768", np.round(g.normal(size=32768) * 8) / 8, 0, 32640, [1, 4096, 32639]))
    cases.append(("normal-16384", g.normal(size=16384), 0, 16320, [1024, 16319]))
    cases.append(("ragged-16385", g.normal(size=16385), 3, 16385, [5, 8000]))
    cases.append(("all-equal-20000", np.full(20000, -1.5), 100, 19900, [1, 9999, 19799]))
    # sizes just past 4096, 8192 and 32768 positions (partly filled last chunk rounds)
    cases.append(("ragged-4097", g.normal(size=4097), 0, 4097, [1, 2048, 4096]))
    cases.append(("ragged-8193", g.normal(size=8193), 100, 8100, [1, 4000, 7999]))
    cases.append(("ragged-32767", np.round(g.normal(size=32767) * 16) / 16, 0, 32700, [1, 16000, 32699]))
    cases.append(("ragged-32769", g.normal(size=32769), 0, 32769, [1, 4096, 32768]))
    # more positions than 64 chunks hold in registers: keys are re-read in every pass
    cases.append(("beyond-registers-140001", g.normal(size=140001), 0, 139000, [1, 4096, 100000]))
    return cases


@pytest.mark.parametrize("case", _select_cases(), ids=lambda c: c[0])
def test_select_edge_cases(case):
    binding = require_gpu()
    import torch
    name, s, b, e, ks = case
    s32 = torch.from_numpy(s.astype(np.float32)).cuda()
    s_exact = s.astype(np.float32).astype(np.float64)
    for k in ks:
        log(f"[select {name}] n={len(s)} doc=[{b},{e}) k={k}")
        kept = binding.tg_select_topk(s32, b, e, k)
        binding.tg_select_check(binding.select_workspace(len(s), "cuda"))
        assert np.array_equal(kept.cpu().numpy().astype(np.int64), oracle.select_topk(s_exact, b, e, k))


@pytest.mark.parametrize("n", [3000, 16384, 32768])
def test_select_unaligned_scores(n):
    """Scores that start 4 bytes past a 16-byte boundary select the same positions as the
    oracle; random-K at the same sizes and spans too."""
    binding = require_gpu()
    import torch
    g = np.random.default_rng(n)
    s = np.round(g.normal(size=n) * 32) / 32
    buf = torch.from_numpy(np.concatenate([[0.0], s]).astype(np.float32)).cuda()
    s32 = buf[1:]
    assert s32.data_ptr() % 16 == 4
    for b, e, k in ((0, n - 64, n // 16), (7, n, 1), (n // 3, 2 * n // 3, n // 10)):
        log(f"[select unaligned] n={n} doc=[{b},{e}) k={k}")
        kept = binding.tg_select_topk(s32, b, e, k)
        binding.tg_select_check(binding.select_workspace(n, "cuda"))
        assert np.array_equal(kept.cpu().numpy().astype(np.int64), oracle.select_topk(s, b, e, k))
        rk = binding.tg_select_random(n, b, e, k, seed=n + k)
        assert np.array_equal(rk.cpu().numpy().astype(np.int64), oracle.select_random(n, b, e, k, n + k))


def test_select_workspace_reuse_across_sizes():
    binding = require_gpu()
    import torch
    g = np.random.default_rng(8)
    ws = torch.zeros(binding.tg_select_workspace_bytes(200000), dtype=torch.uint8, device="cuda")
    for n, q in ((200000, 16), (3000, 16), (77, 16), (150000, 1), (3000, 16), (140000, 64), (32768, 4)):
        s = np.round(g.normal(size=n) * q) / q
        k = int(g.integers(1, n - 10))
        st = torch.from_numpy(s.astype(np.float32)).cuda()
        kept = binding.tg_select_topk(st, 5, n - 5, k, workspace=ws)
        assert np.array_equal(kept.cpu().numpy().astype(np.int64), oracle.select_topk(s, 5, n - 5, k))
        ks = [k, max(1, k // 3)]
        for kk, lst in zip(ks, binding.tg_select_topk_multi(st, 5, n - 5, ks, workspace=ws)):
            assert np.array_equal(lst.cpu().numpy().astype(np.int64), oracle.select_topk(s, 5, n - 5, kk))
    binding.tg_select_check(ws)
    assert_workspace_clean(ws)


def assert_workspace_clean(ws):
    """The parts of a selection workspace that must start at zero are zero again: the head
    (barrier and exit counters, failure word, spin bound, candidate count: bytes 0..19), the
    several-budget kernel's digit histograms (bytes 64 .. 106560: 2048 bins shared, then
    2048 and 1024 bins for each of up to 8 budgets), the one-budget kernel's coarse, fine and
    two digit histograms (bytes 110848 .. 181504: 256 + 16384 + 512 + 512 bins) and the ready
    flags of its 64 chunks (the first word of each 128-byte line from byte 181504)."""
    assert int(ws[:20].count_nonzero()) == 0
    assert int(ws[64:106560].count_nonzero()) == 0
    assert int(ws[110848:181504].count_nonzero()) == 0
    ready = ws[181504:181504 + 64 * 128].view(64, 128)[:, :4]
    assert int(ready.count_nonzero()) == 0


# --------------------------------------------------------------------------- scorer
@pytest.mark.parametrize("n,d_model,d_hidden,ldx", [
    (1, 64, 64, 64), (255, 128, 128, 128), (257, 256, 256, 320), (1000, 2048, 256, 2048), (3001, 512, 64, 576),
    (777, 256, 192, 256), (1000, 2048, 192, 2112),
])
def test_score_bf16_shapes(n, d_model, d_hidden, ldx):
    binding = require_gpu()
    import torch
    g = np.random.default_rng(n + d_hidden)
    xf = g.normal(size=(n, ldx)).astype(np.float32)
    w1f = (g.normal(size=(d_hidden, d_model)) / np.sqrt(d_model)).astype(np.float32)
    w2f = (g.normal(size=d_hidden) / np.sqrt(d_hidden)).astype(np.float32)
    b1 = g.normal(size=d_hidden).astype(np.float32) * 0.3
    xb, w1b, w2b = (inputs.f32_to_bf16_bits(a) for a in (xf, w1f, w2f))
    xt = binding.to_device(xb, "bf16")[:, :d_model]        # row stride ldx
    log(f"[score bf16] n={n} d_model={d_model} d_hidden={d_hidden} ldx={ldx}")
    s = binding.tg_gate_score(xt, binding.to_device(w1b, "bf16"), binding.to_device(w2b, "bf16"),
                              torch.from_numpy(b1).cuda(), 0.375)
    ref = oracle.gate_score(inputs.to_f64(xb, "bf16")[:, :d_model], inputs.to_f64(w1b, "bf16"), b1,
                            inputs.to_f64(w2b, "bf16"), 0.375)
    err = np.abs(s.cpu().numpy() - ref).max()
    log(f"  max_abs={err:.3e}")
    assert err <= SCORE_TOL["bf16"]


@pytest.mark.parametrize("n,d_model,d_hidden", [(1, 4, 1), (100, 36, 7), (513, 256, 64), (64, 1024, 256)])
def test_score_f32_shapes(n, d_model, d_hidden):
    binding = require_gpu()
    import torch
    g = np.random.default_rng(n * 3 + d_hidden)
    x = g.normal(size=(n, d_model)).astype(np.float32)
    w1 = (g.normal(size=(d_hidden, d_model)) / np.sqrt(d_model)).astype(np.float32)
    w2 = g.normal(size=d_hidden).astype(np.float32)
    b1 = g.normal(size=d_hidden).astype(np.float32)
    log(f"[score f32] n={n} d_model={d_model} d_hidden={d_hidden}")
    s = binding.tg_gate_score(torch.from_numpy(x).cuda(), torch.from_numpy(w1).cuda(), torch.from_numpy(w2).cuda(),
                              torch.from_numpy(b1).cuda(), -0.5)
    ref = oracle.gate_score(x, w1, b1, w2, -0.5)
    assert np.abs(s.cpu().numpy() - ref).max() <= SCORE_TOL["f32"]


# --------------------------------------------------------------------------- gather
@pytest.mark.parametrize("dtype,d_model,m", [("bf16", 2048, 1), ("bf16", 2048, 1001), ("bf16", 10, 33),
                                             ("f32", 256, 77), ("f32", 5, 9),
                                             # 8 rows per workgroup from 8192 rows: exact, ragged tails,
                                             # rows narrower than the workgroup
                                             ("bf16", 2048, 8192), ("bf16", 2048, 8197), ("f32", 256, 8195),
                                             ("bf16", 64, 9003)])
def test_gather_shapes(dtype, d_model, m):
    binding = require_gpu()
    import torch
    g = np.random.default_rng(m + d_model)
    n = 3 * m + 5
    xf = g.normal(size=(n, d_model)).astype(np.float32)
    xh = inputs.f32_to_bf16_bits(xf) if dtype == "bf16" else xf
    kept = np.sort(g.choice(n, m, replace=False)).astype(np.int32)
    s = g.normal(size=n).astype(np.float32)
    log(f"[gather {dtype}] d_model={d_model} m={m}")
    xk, sk = binding.tg_gather_kept(binding.to_device(xh, dtype), torch.from_numpy(kept).cuda(),
                                    torch.from_numpy(s).cuda())
    assert np.array_equal(binding.to_host_bits(xk), xh[kept])
    assert np.array_equal(sk.cpu().numpy(), s[kept])


# --------------------------------------------------------------------------- attention
ATTN_CASES = [
    # dtype, m, hq, hkv, d, bias, gapped positions
    ("bf16", 1, 16, 8, 128, True, False),
    ("bf16", 37, 4, 4, 64, True, True),
    ("bf16", 64, 8, 2, 128, True, False),
    ("bf16", 65, 8, 1, 64, True, True),
    ("bf16", 200, 2, 1, 128, False, False),
    ("bf16", 333, 16, 8, 128, True, True),
    ("bf16", 517, 6, 3, 64, True, False),
    ("bf16", 1088, 16, 8, 128, True, True),
    ("f32", 1, 4, 2, 64, True, False),
    ("f32", 70, 4, 2, 64, True, True),
    ("f32", 130, 3, 1, 128, False, False),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c)))
def test_attention_shapes(case):
    binding = require_gpu()
    import torch
    dtype, m, hq, hkv, d, bias, gapped = case
    g = np.random.default_rng(m * 7 + hq + d)
    store = (lambda a: inputs.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    q = store(g.normal(size=(m, hq, d)).astype(np.float32))
    k = store(g.normal(size=(m, hkv, d)).astype(np.float32))
    v = store(g.normal(size=(m, hkv, d)).astype(np.float32))
    pos = (np.sort(g.choice(5 * m + 3, m, replace=False)) if gapped else np.arange(m)).astype(np.int32)
    s = (g.normal(size=m) * 2).astype(np.float32)
    gain = g.uniform(0.5, 1.5, size=hq).astype(np.float32)
    tau = 1.15
    log(f"[attention {dtype}] m={m} hq={hq} hkv={hkv} d={d} bias={bias} gapped={gapped}")
    o = binding.tg_gated_attention(binding.to_device(q, dtype), binding.to_device(k, dtype),
                                   binding.to_device(v, dtype), torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(s).cuda() if bias else None,
                                   torch.from_numpy(gain).cuda() if bias else None, tau)
    torch.cuda.synchronize()
    ref = oracle.gated_attention(inputs.to_f64(q, dtype), inputs.to_f64(k, dtype), inputs.to_f64(v, dtype), pos,
                                 s if bias else None, gain if bias else None, tau)
    err = np.abs(host_f64(o) - ref)
    log(f"  max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= ATTN_MAX_TOL[dtype] and err.mean() <= ATTN_MEAN_TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_positions_near_int32_max(dtype):
    """Gapped positions within 10^6 of the int32 limit: the causal mask compares them as
    int32 (no overflow in the kernels' position handling)."""
    binding = require_gpu()
    import torch
    m, hq, hkv, d = 333, 8, 2, 128 if dtype == "bf16" else 64
    g = np.random.default_rng(2**31 - 1)
    store = (lambda a: inputs.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    q = store(g.normal(size=(m, hq, d)).astype(np.float32))
    k = store(g.normal(size=(m, hkv, d)).astype(np.float32))
    v = store(g.normal(size=(m, hkv, d)).astype(np.float32))
    pos = np.sort(g.choice(np.arange(2**31 - 10**6, 2**31 - 1), m, replace=False)).astype(np.int32)
    s = (g.normal(size=m) * 2).astype(np.float32)
    gain = g.uniform(0.5, 1.5, size=hq).astype(np.float32)
    log(f"[attention {dtype}, positions near 2^31] m={m} hq={hq} hkv={hkv} d={d} pos {pos[0]}..{pos[-1]}")
    o = binding.tg_gated_attention(binding.to_device(q, dtype), binding.to_device(k, dtype),
                                   binding.to_device(v, dtype), torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(s).cuda(), torch.from_numpy(gain).cuda(), 1.05)
    torch.cuda.synchronize()
    ref = oracle.gated_attention(inputs.to_f64(q, dtype), inputs.to_f64(k, dtype), inputs.to_f64(v, dtype), pos,
                                 s, gain, 1.05)
    err = np.abs(host_f64(o) - ref)
    log(f"  max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= ATTN_MAX_TOL[dtype] and err.mean() <= ATTN_MEAN_TOL[dtype]


def test_attention_first_row_is_its_own_value():
    """Row 0 sees one key, so its output is V_0 rounded -- exact on the GPU too."""
    binding = require_gpu()
    import torch
    g = np.random.default_rng(11)
    m, hq, hkv, d = 300, 16, 8, 128
    q, k, v = (inputs.f32_to_bf16_bits(g.normal(size=(m, h, d)).astype(np.float32)) for h in (hq, hkv, hkv))
    o = binding.tg_gated_attention(binding.to_device(q, "bf16"), binding.to_device(k, "bf16"),
                                   binding.to_device(v, "bf16"), None, torch.zeros(m, device="cuda"),
                                   torch.ones(hq, device="cuda"), 0.9)
    assert np.array_equal(binding.to_host_bits(o)[0], np.repeat(v[0], hq // hkv, axis=0))
