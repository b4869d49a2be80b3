"""The seeded input generators: rounding, determinism and the planted spans."""
import numpy as np
import torch

from learned_token_pruning_scorer_amd import configs, inputs


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.normal(size=100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, -1e-40,
                  1.00390625, 1.01171875, 1.0078125], dtype=np.float32),
    ])
    bits = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    # widening is exact: re-rounding a widened value is the identity
    assert np.array_equal(inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(bits)), bits)
    nan_bits = inputs.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(inputs.bf16_bits_to_f32(nan_bits)[0])


def test_generators_are_deterministic_and_shaped():
    w = configs.WORKLOADS["tiny"]
    a, b = inputs.gate_inputs(w), inputs.gate_inputs(w)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w1, b.w1) and np.array_equal(a.w2, b.w2)
    assert a.x.shape == (w.n, w.d_model) and a.x.dtype == np.float32
    assert a.w1.shape == (w.d_hidden, w.d_model)
    kept = np.arange(w.n_kept(w.budgets[0]))
    at = inputs.attention_inputs(w, kept)
    assert at.q.shape == (len(kept), w.n_q_heads, w.head_dim)
    assert at.k.shape == (len(kept), w.n_kv_heads, w.head_dim)
    assert np.all((at.gain >= 0.5) & (at.gain <= 1.5))


def test_spans_are_disjoint_and_inside_the_document():
    for name in ("niah16k", "mdqa32k", "long128k", "sweep64k"):
        w = configs.WORKLOADS[name]
        st = inputs.span_starts(w)
        assert len(st) == w.n_spans
        assert np.all(st >= w.doc_begin) and np.all(st + w.span_len <= w.doc_end)
        assert np.all(np.diff(st) >= w.span_len)


def test_sample_rows_forces_rows_and_is_sorted():
    r = inputs.sample_rows(1000, 256, forced=(0, 999, 640), seed=0)
    assert len(r) == 256 and np.all(np.diff(r) > 0)
    assert {0, 999, 640} <= set(r.tolist())
    assert np.array_equal(r, inputs.sample_rows(1000, 256, forced=(0, 999, 640), seed=0))


def test_sweep_rows_are_shared_across_budgets():
    # rows drawn per position: the same kept position gets the same vectors
    w = configs.WORKLOADS["sweep64k"]
    small = configs.Workload(**{**w.__dict__, "n": 300, "n_question": 4, "n_spans": 0, "span_len": 0,
                                "span_shift": 0.0, "head_dim": 8, "n_q_heads": 2, "n_kv_heads": 1,
                                "d_model": 16, "d_hidden": 8})
    a = inputs.attention_inputs(small, np.array([0, 5, 9, 299]))
    b = inputs.attention_inputs(small, np.array([5, 299]))
    assert np.array_equal(a.q[[1, 3]], b.q) and np.array_equal(a.v[[1, 3]], b.v)
