#!/usr/bin/env python3
"""Throughput of the TokenGate gated-prefill hot path on one MI355X.

One step = the whole path over one prompt already resident in HBM:
    tg_gate_score (N rows) -> tg_select_topk -> tg_gather_kept -> tg_gated_attention_split (M rows)
(the gated attention with the library's own launch plan: at long contexts it is the plain
tg_gated_attention kernel).  The four launches of a step are captured once in a HIP graph
(torch.cuda.CUDAGraph over the library's calls) and replayed: `value` = prompt tokens per
second = N / (wall time of one step), K replays timed back-to-back between two device
synchronisations (warm caches: nothing is flushed between replays; `cold_ms_per_step` is
the same step after a 1 GiB fill).  Per-stage times come from HIP events recorded on the
launch stream inside K eager steps of the same path.

Prints ONE JSON line.  Inputs are seeded synthetic tensors of the workload's
shape (no dataset, no trained weights): see learned_token_pruning_scorer_amd/inputs.py.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# The CPU baseline's BLAS threads: the host cores this process may use, fixed before NumPy
# loads its BLAS (a value already in the environment, e.g. the GPU machine's own, is kept).
_HOST_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(_HOST_CORES))

import numpy as np   # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gated-prefill input tokens/s at 16k/128k; attn TFLOP/s and select GB/s vs peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
CALIB_BYTES = 1 << 30          # streaming copy in --profile-steps mode: reads and writes this many bytes
STAGES = ("score", "select", "gather", "attention")   # the step's launches, in order
# HBM bytes per launch of the attention kernel on long128k, from rocprofv3 FETCH_SIZE and WRITE_SIZE
# scaled by the same counters' reading of the calibration copy (profiles/long128k_hbm_counters.md).
# Reported only while the kernel source is the one the counters were taken on.
ATTN_TRAFFIC = {"workload": "long128k", "bytes": 116849680,
                "source": "learned_token_pruning_scorer_amd/csrc/tg_attention.hip",
                "sha256": "4b3e2e9612150eb779f62a79a73930e8f5637608f32ae5872c4946d393a8b659"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long128k")
    ap.add_argument("--also", default="niah16k,mdqa32k",
                    help="comma-separated workloads reported beside the main one ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-score-rows", type=int, default=131072)
    ap.add_argument("--cpu-attn-rows", type=int, default=0, help="query rows of the CPU attention sample (0 = all)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 64k budget sweep against unpruned attention")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the timings of the attention backward and the multi-budget / random selectors")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip timing the library GEMM and torch's causal attention at the step's shapes")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="if > 0: run only this many steps of the main workload (and as many calls of "
                         "each row timed by --no-next's rows), then one streaming copy of CALIB_BYTES "
                         "(the scale for HBM byte counters); no JSON (for rocprofv3)")
    return ap.parse_args()


def algorithmic(w, k):
    """Algorithmic bytes / flops of one step's stages."""
    m = w.n_kept(k)
    esz = 2 if w.dtype == "bf16" else 4
    score_bytes = w.n * w.d_model * esz + w.d_hidden * w.d_model * esz + w.n * 4
    score_flops = 2.0 * w.n * w.d_model * w.d_hidden
    select_bytes = w.n * 4 + m * 4
    gather_bytes = 2 * m * w.d_model * esz + m * 4 + 2 * m * 4
    attn_flops = 4.0 * w.head_dim * w.n_q_heads * m * (m + 1) / 2
    return dict(m=m, score_bytes=score_bytes, score_flops=score_flops, select_bytes=select_bytes,
                gather_bytes=gather_bytes, select_gather_bytes=select_bytes + gather_bytes, attn_flops=attn_flops)


class Path:
    """Device-resident inputs and preallocated outputs of one workload."""

    def __init__(self, name, binding, torch, k=None, gi=None, full_qkv=None):
        """gi: the workload's gate inputs if already generated; full_qkv: device Q/K/V of every
        prompt position (workloads that draw them per position), gathered here by the kept rows."""
        from learned_token_pruning_scorer_amd import configs, inputs
        self.b, self.torch = binding, torch
        self.w = w = configs.WORKLOADS[name]
        self.k = k if k is not None else (w.budgets[0] if len(w.budgets) == 1 else w.budgets[-1])
        self.gi = gi = gi if gi is not None else inputs.gate_inputs(w)
        dev = "cuda"
        self.x = binding.to_device(gi.x, w.dtype, dev)
        self.w1 = binding.to_device(gi.w1, w.dtype, dev)
        self.w2 = binding.to_device(gi.w2, w.dtype, dev)
        self.b1 = torch.from_numpy(gi.b1).to(dev)
        self.m = m = w.n_kept(self.k)
        self.scores = torch.empty(w.n, dtype=torch.float32, device=dev)
        self.kept = torch.empty(m, dtype=torch.int32, device=dev)
        self.ws = torch.zeros(binding.tg_select_workspace_bytes(w.n), dtype=torch.uint8, device=dev)
        self.xk = torch.empty(m, w.d_model, dtype=self.x.dtype, device=dev)
        self.sk = torch.empty(m, dtype=torch.float32, device=dev)
        # Q/K/V of the kept rows (their projection from hidden states is not part of the path)
        binding.tg_gate_score(self.x, self.w1, self.w2, self.b1, gi.b2, out=self.scores)
        binding.tg_select_topk(self.scores, w.doc_begin, w.doc_end, self.k, out=self.kept, workspace=self.ws)
        binding.tg_select_check(self.ws)
        if full_qkv is not None:
            idx = self.kept.long()
            self.q, self.kk, self.v = (t.index_select(0, idx).contiguous() for t in full_qkv)
            self.gain = torch.from_numpy(inputs.gains(w)).to(dev)
            self.tau = w.tau
        else:
            ai = inputs.attention_inputs(w, self.kept.cpu().numpy())
            self.q = binding.to_device(ai.q, w.dtype, dev)
            self.kk = binding.to_device(ai.k, w.dtype, dev)
            self.v = binding.to_device(ai.v, w.dtype, dev)
            self.gain = torch.from_numpy(ai.gain).to(dev)
            self.tau = ai.tau
        self.o = torch.empty_like(self.q)
        hq, hkv, d = self.q.shape[1], self.kk.shape[1], self.q.shape[2]
        self.attn_ws_bytes = binding.tg_gated_attention_split_workspace_bytes(m, hq, hkv, d, 0)
        self.attn_ws = torch.empty(max(256, self.attn_ws_bytes), dtype=torch.uint8, device=dev)

    def attention(self, out=None, s_kept="kept", gain="kept", tau=None):
        s_kept = self.sk if s_kept == "kept" else s_kept
        gain = self.gain if gain == "kept" else gain
        self.b.tg_gated_attention_split(self.q, self.kk, self.v, self.kept, s_kept, gain,
                                        self.tau if tau is None else tau, out=self.o if out is None else out,
                                        workspace=self.attn_ws)

    def step(self, ev=None):
        b, w = self.b, self.w
        if ev: ev[0].record()
        b.tg_gate_score(self.x, self.w1, self.w2, self.b1, self.gi.b2, out=self.scores)
        if ev: ev[1].record()
        b.tg_select_topk(self.scores, w.doc_begin, w.doc_end, self.k, out=self.kept, workspace=self.ws)
        if ev: ev[2].record()
        b.tg_gather_kept(self.x, self.kept, self.scores, out=self.xk, s_out=self.sk)
        if ev: ev[3].record()
        self.attention()
        if ev: ev[4].record()

    def graph(self):
        """The step captured in a HIP graph (after warm-up launches on a side stream)."""
        if getattr(self, "_graph", None) is None:
            torch = self.torch
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for _ in range(2):
                    self.step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            self._graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self._graph):
                self.step()
            torch.cuda.synchronize()
        return self._graph

    def timed_graph(self, steps, warmup):
        """Wall time per step of `steps` graph replays, after `warmup` untimed ones."""
        torch = self.torch
        g = self.graph()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def timed_cold(self, reps):
        """Median time of a replayed step with the caches flushed before it: a 1 GiB fill (outside
        the events) evicts the L2s and the 256 MB Infinity Cache, so X comes from HBM."""
        torch = self.torch
        g = self.graph()
        flush = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            flush.zero_()
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        del flush
        return float(np.median([a.elapsed_time(b) for a, b in evs])) / 1e3

    def timed(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        self.b.tg_select_check(self.ws)
        stage = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(STAGES))] for e in evs]) * 1e3   # us
        # step period on the GPU timeline (start of one step to the start of the next), median:
        # robust to a host hiccup, which the wall-clock mean is not
        period = [evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(steps - 1)] or [wall * 1e3]
        self.eager_period = float(np.median(period)) / 1e3
        return wall / steps, stage.mean(axis=0), np.median(stage, axis=0)


def attention_traffic(workload):
    """Counter-measured HBM bytes per attention launch, or None if stale or for another workload."""
    import hashlib
    if workload != ATTN_TRAFFIC["workload"]:
        return None
    try:
        with open(os.path.join(ROOT, ATTN_TRAFFIC["source"]), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return ATTN_TRAFFIC["bytes"] if digest == ATTN_TRAFFIC["sha256"] else None


def _event_time_us(torch, fn, reps, warmup=3):
    """Mean time of fn() from HIP events on the current stream (the stream the bindings launch on)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3


def next_rows(path, reps):
    """Timings of the rows beyond the forward step, on the main workload's tensors:
    the attention backward, several budgets in one select, and the random-K selector."""
    torch, b, w = path.torch, path.b, path.w
    res = {}
    # attention backward: algorithmic flops = five causal products (S, dP, dQ, dK, dV) of the
    # forward's per-product size; the kernels recompute S and dP once more for dQ
    g = torch.Generator(device="cuda").manual_seed(1)
    dout = torch.randn(path.q.shape, generator=g, device="cuda", dtype=torch.float32).to(path.q.dtype)
    out, lse = b.tg_gated_attention_lse(path.q, path.kk, path.v, path.kept, path.sk, path.gain, path.tau)
    ws = torch.empty(max(256, int(b.lib.tg_gated_attention_backward_workspace_bytes(
        path.m, w.n_q_heads, w.n_kv_heads, w.head_dim))), dtype=torch.uint8, device="cuda")
    us = _event_time_us(torch, lambda: b.tg_gated_attention_backward(
        path.q, path.kk, path.v, path.kept, path.sk, path.gain, path.tau, out, lse, dout, workspace=ws), reps)
    flops = 2.5 * algorithmic(w, path.k)["attn_flops"]
    res["attention_backward"] = {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                                 "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                                 "flops": flops, "note": "five causal products of size 2 M^2 d Hq / 2"}
    us_fwd = _event_time_us(torch, lambda: b.tg_gated_attention_lse(
        path.q, path.kk, path.v, path.kept, path.sk, path.gain, path.tau, out=out, lse=lse), reps)
    res["attention_forward_with_lse"] = {"us": us_fwd}
    # the same selection and gather in one launch (tg_select_gather, the allocation-free path's kernel)
    kept2 = torch.empty_like(path.kept)
    xk2, sk2 = torch.empty_like(path.xk), torch.empty_like(path.sk)
    us = _event_time_us(torch, lambda: b.tg_select_gather(path.scores, path.x, w.doc_begin, w.doc_end, path.k,
                                                          kept=kept2, x_kept=xk2, s_kept=sk2, workspace=path.ws), reps)
    byts = algorithmic(w, path.k)["select_gather_bytes"]
    res["select_gather_one_launch"] = {"us": us, "frac_hbm_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                       "note": "tg_select_gather (selection and row gather fused) on the step's inputs"}
    del kept2, xk2, sk2
    # several budgets over one histogram of the same scores
    ks = [path.k // 8, path.k // 4, path.k // 2, path.k]
    outs = torch.empty(sum(w.n_kept(k) for k in ks), dtype=torch.int32, device="cuda")
    us = _event_time_us(torch, lambda: b.tg_select_topk_multi(path.scores, w.doc_begin, w.doc_end, ks, out=outs,
                                                               workspace=path.ws), reps)
    byts = w.n * 4 + sum(w.n_kept(k) for k in ks) * 4
    res["select_topk_multi"] = {"budgets": ks, "us": us, "gbs": byts / (us * 1e-6) / 1e9,
                                "frac_hbm_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "bytes": byts}
    # kept-row projection + rotary + KV emission: 2 M d_model (Hq + 2 Hkv) d flops
    from learned_token_pruning_scorer_amd import inputs
    wq = b.to_device(inputs.qkv_weights(w), w.dtype, "cuda")
    qo = torch.empty_like(path.q)
    kc, vc = torch.empty_like(path.kk), torch.empty_like(path.v)
    pc = torch.empty(path.m, dtype=torch.int32, device="cuda")
    qws = torch.empty(max(256, int(b.lib.tg_qkv_rope_workspace_bytes(path.m, w.head_dim))), dtype=torch.uint8,
                      device="cuda")
    us = _event_time_us(torch, lambda: b.tg_qkv_rope(path.xk, wq, path.kept, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                                     inputs.ROPE_THETA, q_out=qo, k_cache=kc, v_cache=vc,
                                                     pos_cache=pc, workspace=qws), reps)
    flops = 2.0 * path.m * w.d_model * (w.n_q_heads + 2 * w.n_kv_heads) * w.head_dim
    res["qkv_rope"] = {"us": us, "tflops": flops / (us * 1e-6) / 1e12,
                       "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, "flops": flops}
    del wq, qo, kc, vc, pc, qws
    # the key bias's cost: the same attention with s_kept = gain = NULL
    us_on = _event_time_us(torch, lambda: path.attention(), reps)
    us_off = _event_time_us(torch, lambda: path.attention(s_kept=None, gain=None), reps)
    res["attention_bias_cost"] = {"us_bias_on": us_on, "us_bias_off": us_off, "ratio": us_on / us_off}
    # one GPU's share in the head-parallel design over 8 GPUs: one K/V head and its query heads
    group = w.n_q_heads // w.n_kv_heads
    qs = path.q[:, :group].contiguous()
    ks_, vs_ = path.kk[:, :1].contiguous(), path.v[:, :1].contiguous()
    gs = path.gain[:group].contiguous()
    os_ = torch.empty_like(qs)
    sws = torch.empty(max(256, b.tg_gated_attention_split_workspace_bytes(path.m, group, 1, w.head_dim, 0)),
                      dtype=torch.uint8, device="cuda")
    us_plain = _event_time_us(torch, lambda: b.tg_gated_attention(qs, ks_, vs_, path.kept, path.sk, gs, path.tau,
                                                                  out=os_), reps)
    us = _event_time_us(torch, lambda: b.tg_gated_attention_split(qs, ks_, vs_, path.kept, path.sk, gs, path.tau,
                                                                  out=os_, workspace=sws), reps)
    flops = 4.0 * w.head_dim * group * path.m * (path.m + 1) / 2
    res["attention_head_shard"] = {"n_q_heads": group, "n_kv_heads": 1, "m": path.m, "us": us,
                                   "us_without_key_split": us_plain,
                                   "tflops": flops / (us * 1e-6) / 1e12,
                                   "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    del qs, ks_, vs_, gs, os_, sws
    kept_r = torch.empty(path.m, dtype=torch.int32, device="cuda")
    us = _event_time_us(torch, lambda: b.tg_select_random(w.n, w.doc_begin, w.doc_end, path.k, 12345,
                                                          out=kept_r, workspace=path.ws), reps)
    res["select_random"] = {"k": path.k, "us": us, "gbs": path.m * 4 / (us * 1e-6) / 1e9, "bytes": path.m * 4}
    del dout, out, lse, ws
    torch.cuda.empty_cache()
    return res


def calibration(path, reps):
    """Library kernels at the step's own shapes, timed beside ours in the same process, as
    context for the roofline fractions: the scorer's product X . W1^T as a plain library GEMM
    (torch.nn.functional.linear, bf16 out, no activation, no 1-wide output), and torch's own
    causal attention (scaled_dot_product_attention, flash backend, no key bias, K/V heads
    expanded to the query heads) on the step's Q/K/V."""
    torch, b, w = path.torch, path.b, path.w
    res = {}
    try:
        ours = _event_time_us(torch, lambda: b.tg_gate_score(path.x, path.w1, path.w2, path.b1, path.gi.b2,
                                                            out=path.scores), reps)
        lib = _event_time_us(torch, lambda: torch.nn.functional.linear(path.x, path.w1), reps)
        res["scorer_vs_library_gemm"] = {"us_scorer": ours, "us_library_gemm": lib, "ratio": ours / lib,
                                         "note": "library GEMM = torch.nn.functional.linear(X, W1) alone"}
    except Exception as e:   # context only: a library that is missing or fails is reported, not fatal
        res["scorer_vs_library_gemm"] = {"error": str(e)[:200]}
    try:
        import torch.nn.functional as F
        from torch.nn.attention import SDPBackend, sdpa_kernel
        group = w.n_q_heads // w.n_kv_heads
        qt = path.q.transpose(0, 1).unsqueeze(0).contiguous()
        kt = path.kk.transpose(0, 1).repeat_interleave(group, dim=0).unsqueeze(0).contiguous()
        vt = path.v.transpose(0, 1).repeat_interleave(group, dim=0).unsqueeze(0).contiguous()
        ours = _event_time_us(torch, lambda: path.attention(), reps)
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            lib = _event_time_us(torch, lambda: F.scaled_dot_product_attention(qt, kt, vt, is_causal=True), reps)
        res["attention_vs_torch_sdpa"] = {"us_gated_attention": ours, "us_torch_sdpa_flash_causal": lib,
                                          "ratio": ours / lib, "m": path.m,
                                          "note": "torch SDPA without the key bias or temperature"}
        del qt, kt, vt
    except Exception as e:
        res["attention_vs_torch_sdpa"] = {"error": str(e)[:200]}
    torch.cuda.empty_cache()
    return res


def sweep64k(binding, torch, steps, warmup):
    """Budget reuse at 64k: the whole path at each budget against unpruned causal attention
    over all N rows (bias off, tau = 1), the comparison the pruning is for."""
    from learned_token_pruning_scorer_amd import configs, inputs
    w = configs.WORKLOADS["sweep64k"]
    out = {"workload": w.name, "n": w.n, "points": []}
    gi = inputs.gate_inputs(w)
    ai = inputs.attention_inputs(w, np.arange(w.n))   # Q/K/V of every position (the unpruned run's)
    full = tuple(binding.to_device(a, w.dtype, "cuda") for a in (ai.q, ai.k, ai.v))
    del ai
    x_bytes = w.n * w.d_model * 2

    def window():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        return torch.cuda.memory_allocated()

    for k in w.budgets:
        # peak device bytes of the pruned path: its own tensors (X, gate weights, scores, kept list,
        # workspaces, gathered rows, the kept rows' Q/K/V, output) allocated and one step run
        # inside the window
        base = window()
        p = Path(w.name, binding, torch, k=k, gi=gi, full_qkv=full)
        p.step()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        _, st, _ = p.timed(steps, warmup)
        sec_e = p.eager_period
        sec = p.timed_graph(steps, warmup)
        out["points"].append({"k": k, "m": p.m, "ms_per_step": sec * 1e3, "eager_ms_per_step": sec_e * 1e3,
                              "peak_bytes": peak,
                              "stage_us_mean": dict(zip(STAGES, (float(v) for v in st)))})
        del p
        torch.cuda.empty_cache()
    # peak device bytes of the unpruned layer: X, Q/K/V of all N rows, output, run once
    base = window()
    xu = binding.to_device(gi.x, w.dtype, "cuda")
    qu, ku, vu = (t.clone() for t in full)
    ou = torch.empty_like(qu)
    wsu = torch.empty(max(256, binding.tg_gated_attention_split_workspace_bytes(w.n, w.n_q_heads, w.n_kv_heads,
                                                                                w.head_dim, 0)),
                      dtype=torch.uint8, device="cuda")
    binding.tg_gated_attention_split(qu, ku, vu, None, None, None, 1.0, out=ou, workspace=wsu)
    torch.cuda.synchronize()
    peak_u = torch.cuda.max_memory_allocated() - base
    del xu, qu, ku, vu, ou, wsu
    torch.cuda.empty_cache()
    out["memory"] = {"unpruned_peak_bytes": peak_u, "x_bytes": x_bytes,
                     "note": "peak device bytes allocated by each path's own tensors over one run; "
                             "ratios with X (the gate layer's input, held by both) counted and excluded"}
    for pt in out["points"]:
        pt["memory_ratio_vs_unpruned"] = peak_u / pt["peak_bytes"]
        pt["memory_ratio_vs_unpruned_excl_x"] = (peak_u - x_bytes) / (pt["peak_bytes"] - x_bytes)
    q, k, v = full
    o = torch.empty_like(q)
    reps = max(3, steps // 4)
    ws = torch.empty(max(256, binding.tg_gated_attention_split_workspace_bytes(w.n, w.n_q_heads, w.n_kv_heads,
                                                                               w.head_dim, 0)),
                     dtype=torch.uint8, device="cuda")
    us = _event_time_us(torch, lambda: binding.tg_gated_attention_split(q, k, v, None, None, None, 1.0, out=o,
                                                                        workspace=ws), reps, warmup=2)
    flops = 4.0 * w.head_dim * w.n_q_heads * w.n * (w.n + 1) / 2
    out["unpruned"] = {"m": w.n, "ms": us / 1e3, "tflops": flops / (us * 1e-6) / 1e12,
                       "frac_mfma_peak": flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    for pt in out["points"]:
        pt["time_ratio_vs_unpruned"] = (us / 1e3) / pt["ms_per_step"]
    del q, k, v, o, full, ws
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(name, score_rows, attn_rows):
    """The float64 oracle on a bounded sample of the same workload, scaled to tokens/s."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    import oracle
    from learned_token_pruning_scorer_amd import configs, inputs
    w = configs.WORKLOADS[name]
    k = w.budgets[0] if len(w.budgets) == 1 else w.budgets[-1]
    gi = inputs.gate_inputs(w)
    g = np.random.default_rng(5)
    rows = np.sort(g.choice(w.n, min(score_rows, w.n), replace=False))
    x64 = inputs.to_f64(gi.x[rows], w.dtype)
    w164, w264 = inputs.to_f64(gi.w1, w.dtype), inputs.to_f64(gi.w2, w.dtype)
    t = time.perf_counter()
    oracle.gate_score(x64, w164, gi.b1, w264, gi.b2)
    t_score = (time.perf_counter() - t) * (w.n / len(rows))
    # selection and gather run on the full workload (scores of all rows are drawn cheaply here:
    # the oracle's own selector is timed, not the scores' provenance)
    s_full = np.random.default_rng(6).normal(size=w.n)
    t = time.perf_counter()
    kept = oracle.select_topk(s_full, w.doc_begin, w.doc_end, k)
    t_select = time.perf_counter() - t
    t = time.perf_counter()
    oracle.gather_kept(gi.x, s_full, kept)
    t_gather = time.perf_counter() - t
    ai = inputs.attention_inputs(w, kept)
    m = len(kept)
    arows = inputs.sample_rows(m, m if attn_rows <= 0 else min(attn_rows, m), forced=(0, m - 1), seed=1)
    q64, k64, v64 = (inputs.to_f64(a, w.dtype) for a in (ai.q, ai.k, ai.v))
    t = time.perf_counter()
    oracle.gated_attention(q64, k64, v64, kept, s_full[kept], ai.gain, ai.tau, rows=arows)
    t_attn_sample = time.perf_counter() - t
    # attention cost of a row grows with the keys it sees: scale by the causal work ratio
    work_sample = float(np.sum(arows + 1))
    work_all = m * (m + 1) / 2.0
    t_attn = t_attn_sample * (work_all / work_sample)
    total = t_score + t_select + t_gather + t_attn
    measured = t_score * (len(rows) / w.n) + t_select + t_gather + t_attn_sample
    return {"value": w.n / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
            "host_cores_available": _HOST_CORES,
            "blas_threads_env": {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")},
            "sample": (f"{name}: gate score on {len(rows)} of {w.n} rows, full select and gather, "
                       f"attention on {len(arows)} of {m} query rows"
                       + ("" if len(rows) == w.n and len(arows) == m else
                          "; each scaled to the full workload (score by rows, attention by causal key count)")
                       + f"; {measured:.1f} s of CPU time measured"),
            "stage_seconds": {"score": t_score, "select": t_select, "gather": t_gather, "attention": t_attn}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported: the path is "
              "implemented for one GPU, and how it would shard over several is a design only", file=sys.stderr)
        return 2
    import torch
    from learned_token_pruning_scorer_amd import binding
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    path = Path(args.workload, binding, torch)
    print(f"[bench] inputs ready: {args.workload}", file=sys.stderr, flush=True)
    if args.profile_steps > 0:
        for _ in range(args.profile_steps):
            path.step()
        torch.cuda.synchronize()
        if not args.no_next:
            next_rows(path, args.profile_steps)
        # a plain streaming copy of known size: its FETCH_SIZE / WRITE_SIZE give the counters' scale
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] profiled {args.profile_steps} steps of {args.workload}", file=sys.stderr, flush=True)
        return 0

    _, stage_mean, stage_med = path.timed(args.steps, args.warmup)
    sec_eager = path.eager_period
    sec = path.timed_graph(args.steps, args.warmup)
    sec_cold = path.timed_cold(max(5, args.steps // 2))
    w = path.w
    alg = algorithmic(w, path.k)
    attn_tflops = alg["attn_flops"] / (stage_mean[3] * 1e-6) / 1e12
    sel_gather_gbs = alg["select_gather_bytes"] / ((stage_mean[1] + stage_mean[2]) * 1e-6) / 1e9
    score_gbs = alg["score_bytes"] / (stage_mean[0] * 1e-6) / 1e9
    score_tflops = alg["score_flops"] / (stage_mean[0] * 1e-6) / 1e12
    print(f"[bench] {args.workload}: {sec * 1e3:.3f} ms/step (graph), {sec_eager * 1e3:.3f} eager; "
          f"stages us (mean) score {stage_mean[0]:.1f} select {stage_mean[1]:.1f} gather {stage_mean[2]:.1f} "
          f"attention {stage_mean[3]:.1f}", file=sys.stderr, flush=True)

    also = []
    for name in [a for a in args.also.split(",") if a and a != args.workload]:
        p2 = Path(name, binding, torch)
        _, st2, st2m = p2.timed(args.steps, args.warmup)
        sec2e = p2.eager_period
        sec2 = p2.timed_graph(args.steps, args.warmup)
        sec2c = p2.timed_cold(max(5, args.steps // 2))
        alg2 = algorithmic(p2.w, p2.k)
        also.append({"workload": name, "n": p2.w.n, "k": p2.k, "m": p2.m, "tokens_per_s": p2.w.n / sec2,
                     "ms_per_step": sec2 * 1e3, "cold_ms_per_step": sec2c * 1e3, "cold_tokens_per_s": p2.w.n / sec2c,
                     "eager_ms_per_step": sec2e * 1e3, "eager_tokens_per_s": p2.w.n / sec2e,
                     "stage_us_mean": dict(zip(STAGES, (float(v) for v in st2))),
                     "stage_us_median": dict(zip(STAGES, (float(v) for v in st2m))),
                     "attention_frac_mfma_peak": alg2["attn_flops"] / (st2[3] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                     "select_gather_frac_hbm_peak":
                         alg2["select_gather_bytes"] / ((st2[1] + st2[2]) * 1e-6) / 1e9 / PEAK_HBM_GBS,
                     "score_frac_hbm_peak": alg2["score_bytes"] / (st2[0] * 1e-6) / 1e9 / PEAK_HBM_GBS})
        print(f"[bench] {name}: {sec2 * 1e3:.3f} ms/step (graph)", file=sys.stderr, flush=True)
        del p2
        torch.cuda.empty_cache()

    nxt = None
    if not args.no_next:
        print("[bench] timing the backward and the selector variants", file=sys.stderr, flush=True)
        nxt = next_rows(path, max(5, args.steps // 2))

    cal = None
    if not args.no_calibration:
        print("[bench] library GEMM and torch attention at the step's shapes", file=sys.stderr, flush=True)
        cal = calibration(path, max(5, args.steps // 2))

    sweep = None
    if not args.no_sweep:
        print("[bench] 64k budget sweep against unpruned attention", file=sys.stderr, flush=True)
        sweep = sweep64k(binding, torch, args.steps, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload, args.cpu_score_rows, args.cpu_attn_rows)

    out = {
        "metric": METRIC,
        "value": w.n / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "eager_ms_per_step": sec_eager * 1e3,
        "cold_ms_per_step": sec_cold * 1e3,
        "step_launch": "HIP graph of the step's four launches (score, select, gather, attention), replayed back "
                       "to back; eager steps give the stage times",
        "value_cache_state": "warm: back-to-back replays, nothing flushed between them (X of the 128k workload, "
                             "512 MiB, exceeds the 256 MB Infinity Cache anyway); cold_ms_per_step = median "
                             "replay after a 1 GiB fill that evicts L2 and the Infinity Cache",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, shaped like the workload; no dataset or trained weights)",
        "config": {"workload": w.name, "n": w.n, "n_doc": w.n_doc, "k": path.k, "m": path.m,
                   "d_model": w.d_model, "d_hidden": w.d_hidden, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "tau": w.tau},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel", "achieved": attn_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": attention_traffic(w.name)},
        "cpu_baseline": cpu,
        "stages": {
            "us_mean": dict(zip(STAGES, (float(v) for v in stage_mean))),
            "us_median": dict(zip(STAGES, (float(v) for v in stage_med))),
            "attention_tflops": attn_tflops, "attention_frac_mfma_peak": attn_tflops / PEAK_BF16_TFLOPS,
            "select_gather_gbs": sel_gather_gbs, "select_gather_frac_hbm_peak": sel_gather_gbs / PEAK_HBM_GBS,
            "select_gather_bytes": alg["select_gather_bytes"],
            "score_gbs": score_gbs, "score_frac_hbm_peak": score_gbs / PEAK_HBM_GBS, "score_tflops": score_tflops,
        },
        "also": also,
        "next_rows": nxt,
        "calibration": cal,
        "sweep64k": sweep,
    }
    print(json.dumps(out), flush=True)
    # release device memory while the runtime is fully up, before interpreter teardown
    del path
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
