"""Seeded synthetic inputs for the gated-prefill path.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
checks.  It holds none of the method's arithmetic: it only draws random
tensors, rounds them to bf16 storage, and plants evidence spans.  Every tensor
comes from its own PCG64 stream, keyed by (seed, stream id):

    0 hidden states X      1 gate W1      3 gate w2      4 span offsets
    5 Q                    6 K            7 V            8 per-head gain
    9 sampled query rows

Recipe (all workloads): X ~ N(0,1); W1 ~ N(0, 1/d_model); w2 ~ N(0, 1/d_hidden);
b1 = 0, b2 = 0; Q, K, V ~ N(0,1); gain ~ U(gain_lo, gain_hi).  bf16 workloads
draw in float32 and round to bf16 with round-to-nearest-even.

Evidence spans ("needles"): the document [0, D) is cut into n_spans equal
segments and one span of span_len tokens is placed at a uniformly drawn offset
inside each, so spans never overlap.  Their rows are shifted by span_shift
along u = W1^T w2 / |W1^T w2| (computed from the stored, rounded weights), the
direction in which a small input change raises the gate's output the most when
the MLP biases are zero, then rounded again.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import Workload

STREAM_X, STREAM_W1, STREAM_W2, STREAM_SPANS = 0, 1, 3, 4
STREAM_Q, STREAM_K, STREAM_V, STREAM_GAIN, STREAM_ROWS = 5, 6, 7, 8, 9
STREAM_WQKV = 10
ROPE_THETA = 1.0e6     # rotary base of the Qwen3 family whose shapes the workloads borrow

_CHUNK_ROWS = 4096   # rows drawn per call; fixed so that streams are reproducible


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream,))))


# ----------------------------------------------------------------------------------------
# bf16 storage helpers (bit patterns held in uint16 arrays)
# ----------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 22
    for i in range(0, flat_u.size, step):
        blk = flat_u[i:i + step]
        r = (blk >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += blk                      # finite values cannot overflow uint32 here
        r >>= np.uint32(16)
        o = r.astype(np.uint16)
        nan = (blk & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            o[nan] = np.uint16(0x7FC0)
        flat_o[i:i + step] = o
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored tensor (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _normal_rows(g: np.random.Generator, rows: int, row_shape: tuple) -> np.ndarray:
    out = np.empty((rows,) + tuple(row_shape), dtype=np.float32)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = g.standard_normal((r1 - r0,) + tuple(row_shape), dtype=np.float32)
    return out


# ----------------------------------------------------------------------------------------
# gate inputs
# ----------------------------------------------------------------------------------------
@dataclass
class GateInputs:
    dtype: str
    x: np.ndarray          # [N, d_model]  bf16 bits (uint16) or float32
    w1: np.ndarray         # [d_hidden, d_model]
    b1: np.ndarray         # [d_hidden] float32
    w2: np.ndarray         # [d_hidden]
    b2: float
    doc_begin: int
    doc_end: int
    span_starts: np.ndarray   # int64 [n_spans]
    span_len: int


def span_starts(w: Workload) -> np.ndarray:
    if w.n_spans == 0:
        return np.zeros(0, dtype=np.int64)
    seg = w.n_doc // w.n_spans
    if seg < w.span_len:
        raise ValueError("spans do not fit in the document")
    g = rng(w.seed, STREAM_SPANS)
    offs = g.integers(0, seg - w.span_len + 1, size=w.n_spans)
    return (w.doc_begin + np.arange(w.n_spans) * seg + offs).astype(np.int64)


def gate_inputs(w: Workload) -> GateInputs:
    w1_32 = _normal_rows(rng(w.seed, STREAM_W1), w.d_hidden, (w.d_model,))
    w1_32 *= np.float32(1.0 / np.sqrt(w.d_model))
    w2_32 = rng(w.seed, STREAM_W2).standard_normal(w.d_hidden, dtype=np.float32)
    w2_32 *= np.float32(1.0 / np.sqrt(w.d_hidden))
    w1 = _store(w1_32, w.dtype)
    w2 = _store(w2_32, w.dtype)
    b1 = np.zeros(w.d_hidden, dtype=np.float32)

    x32 = _normal_rows(rng(w.seed, STREAM_X), w.n, (w.d_model,))
    starts = span_starts(w)
    if len(starts):
        u = to_f64(w1, w.dtype).T @ to_f64(w2, w.dtype)
        u /= np.linalg.norm(u)
        shift = (w.span_shift * u).astype(np.float32)
        for s0 in starts:
            x32[s0:s0 + w.span_len] += shift
    x = _store(x32, w.dtype)
    del x32
    return GateInputs(w.dtype, x, w1, b1, w2, 0.0, w.doc_begin, w.doc_end, starts, w.span_len)


# ----------------------------------------------------------------------------------------
# attention inputs
# ----------------------------------------------------------------------------------------
@dataclass
class AttentionInputs:
    dtype: str
    q: np.ndarray          # [M, Hq, d]
    k: np.ndarray          # [M, Hkv, d]
    v: np.ndarray          # [M, Hkv, d]
    gain: np.ndarray       # [Hq] float32
    tau: float


def gains(w: Workload) -> np.ndarray:
    g = rng(w.seed, STREAM_GAIN)
    return g.uniform(w.gain_lo, w.gain_hi, size=w.n_q_heads).astype(np.float32)


def attention_inputs(w: Workload, kept_idx: np.ndarray) -> AttentionInputs:
    """Q/K/V for the rows above the gate.

    Workloads with a single budget draw Q/K/V directly for the M kept rows.  The
    budget sweep draws them per prompt position and takes the kept rows, so every
    budget and the unpruned run see the same token vectors.
    """
    kept_idx = np.asarray(kept_idx, dtype=np.int64)
    m = len(kept_idx)
    tensors = []
    for stream, heads in ((STREAM_Q, w.n_q_heads), (STREAM_K, w.n_kv_heads), (STREAM_V, w.n_kv_heads)):
        g = rng(w.seed, stream)
        if w.unpruned_reference:
            full = _normal_rows(g, w.n, (heads, w.head_dim))
            t32 = np.ascontiguousarray(full[kept_idx])
            del full
        else:
            t32 = _normal_rows(g, m, (heads, w.head_dim))
        tensors.append(_store(t32, w.dtype))
    return AttentionInputs(w.dtype, tensors[0], tensors[1], tensors[2], gains(w), w.tau)


def sample_rows(m: int, count: int, forced=(), seed: int = 0) -> np.ndarray:
    """Sorted sample of query rows: `forced` rows plus seeded distinct extras."""
    forced = sorted({int(r) for r in forced if 0 <= int(r) < m})
    if count >= m:
        return np.arange(m, dtype=np.int64)
    g = rng(seed, STREAM_ROWS)
    pool = np.setdiff1d(np.arange(m, dtype=np.int64), np.asarray(forced, dtype=np.int64))
    extra = g.choice(pool, size=max(0, count - len(forced)), replace=False)
    return np.sort(np.concatenate([np.asarray(forced, dtype=np.int64), extra]))


def first_question_row(w: Workload, k: int) -> int:
    """Row index (after compaction) of the first question token."""
    return min(k, w.n_doc)


# ----------------------------------------------------------------------------------------
# kept-row projection weights (the step after the gather)
# ----------------------------------------------------------------------------------------
def qkv_weights(w: Workload) -> np.ndarray:
    """W_qkv [(Hq + 2 Hkv) d, d_model] ~ N(0, 1/d_model), stored in the workload dtype."""
    n_feat = (w.n_q_heads + 2 * w.n_kv_heads) * w.head_dim
    w32 = _normal_rows(rng(w.seed, STREAM_WQKV), n_feat, (w.d_model,))
    w32 *= np.float32(1.0 / np.sqrt(w.d_model))
    return _store(w32, w.dtype)
