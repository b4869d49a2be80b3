"""The five synthetic workloads of the gated-prefill path.

Each workload stands in, by shape only, for one of the evaluations the
TokenGate pages describe (needle-in-a-haystack at 16k, multi-document QA,
long-context scale-up to 128k, and budget reuse with one gate).  No dataset,
checkpoint or trained weight is involved: every tensor is drawn from a seeded
generator (see ``inputs.py``).

Shape sources: the model dims are Qwen3-1.7B-like (d_model 2048, 16 query heads,
8 key/value heads, head_dim 128), the model all timings are taken on
(aisight.pl, "TokenGate: Stanford i Berkeley ucza model, ktore tokeny pominac ...",
section "Wyniki"; news.chathome.org TokenGate article, section
"ベンチマークでの TokenGate の性能").  The prompt is a document followed by a
question, and only the document may be pruned (aiproducthub.cn,
"斯坦福伯克利TokenGate 预填充提速11.3倍", section 事件详情).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "f32" or "bf16": storage and MFMA operand type
    n: int                     # prompt tokens N
    n_question: int            # question tokens at the end of the prompt (never pruned)
    d_model: int
    d_hidden: int              # gate MLP hidden width
    budgets: tuple             # document tokens kept (one entry per run)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tau: float                 # attention temperature
    gain_lo: float = 0.5       # per-head gain ~ U(gain_lo, gain_hi)
    gain_hi: float = 1.5
    n_spans: int = 0           # planted evidence spans inside the document
    span_len: int = 0
    span_shift: float = 0.0    # shift along the gate's input direction
    seed: int = 0
    unpruned_reference: bool = False   # also run K = all, bias off, tau = 1
    description: str = ""

    @property
    def doc_begin(self) -> int:
        return 0

    @property
    def doc_end(self) -> int:
        return self.n - self.n_question

    @property
    def n_doc(self) -> int:
        return self.doc_end - self.doc_begin

    def n_kept(self, k: int) -> int:
        """Rows above the gate: every question token plus min(k, D) document tokens."""
        return (self.n - self.n_doc) + min(k, self.n_doc)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", dtype="f32", n=512, n_question=64, d_model=256, d_hidden=64,
        budgets=(128,), n_q_heads=4, n_kv_heads=2, head_dim=64, tau=1.2,
        description="tiny fp32: N=512 (448 doc + 64 question), gate 256->64->1, K=128"),
    "niah16k": Workload(
        name="niah16k", dtype="bf16", n=16384, n_question=64, d_model=2048, d_hidden=256,
        budgets=(1024,), n_q_heads=16, n_kv_heads=8, head_dim=128, tau=1.1,
        n_spans=1, span_len=32, span_shift=3.0,
        description="needle-in-a-haystack shaped, 16k tokens, one 32-token needle, K=1024"),
    "mdqa32k": Workload(
        name="mdqa32k", dtype="bf16", n=32768, n_question=128, d_model=2048, d_hidden=256,
        budgets=(4096,), n_q_heads=16, n_kv_heads=8, head_dim=128, tau=1.1,
        n_spans=8, span_len=64, span_shift=2.0,
        description="multi-document-QA shaped, 32k tokens, 8 evidence spans of 64, K=4096"),
    "long128k": Workload(
        name="long128k", dtype="bf16", n=131072, n_question=64, d_model=2048, d_hidden=256,
        budgets=(8192,), n_q_heads=16, n_kv_heads=8, head_dim=128, tau=1.1,
        n_spans=1, span_len=32, span_shift=3.0,
        description="long-context 128k tokens, one 32-token needle, K=8192"),
    "sweep64k": Workload(
        name="sweep64k", dtype="bf16", n=65536, n_question=64, d_model=2048, d_hidden=256,
        budgets=(2048, 4096, 8192, 16384), n_q_heads=16, n_kv_heads=8, head_dim=128, tau=1.1,
        n_spans=16, span_len=64, span_shift=2.0, unpruned_reference=True,
        description="budget sweep at 64k with one gate, K in {2048,4096,8192,16384} + unpruned"),
}

ORDER = ("tiny", "niah16k", "mdqa32k", "long128k", "sweep64k")
