"""The five synthetic compaction workloads, as structured records.

Each record is one batch of independent per-KV-head compaction problems. The shapes
follow the pages' workloads: Qwen3-family head dimension 128, 8 KV heads, grouped-query
attention with four query heads per KV head, and compaction ratios of 16x and 32x
("Latent Compaction with Test-Time Training", App. A.1 model shapes and App. A.3 budget
definition B = N0 / r; "Compaction" blog, §Fast KV Compaction via Attention Matching,
context-prefill queries with one query per position).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int          # independent head problems in one batch
    d: int              # head dimension
    T: int              # full-cache keys/values per head
    n: int              # reference queries per head
    t: int              # compacted entries per head
    dtype: str          # "f32" or "bf16" (input dtype; accumulation is fp32)
    causal: bool        # query i sits at position i // group and sees keys 0..i // group
    group: int          # query heads per KV head (GQA); queries are position-major
    heads_per_unit: int = 8     # KV heads per layer / document (seeding)
    unit_kind: str = "none"     # "doc", "layer" or "none": what the outer head index counts
    extra_needles: bool = False  # 0.1% further key rows scaled x4
    ridge_lambda: float = 1e-3

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    def visible_pairs_per_head(self) -> int:
        """Query-key pairs that the mask leaves visible in one head problem."""
        if not self.causal:
            return self.n * self.T
        # position p holds `group` queries, each seeing p + 1 keys; positions 0 .. n/group - 1
        P = self.n // self.group
        return self.group * P * (P + 1) // 2

    def visible_pairs(self) -> int:
        return self.heads * self.visible_pairs_per_head()

    def seed_path(self, h: int) -> tuple[int, int, int]:
        """(layer, doc, kv_head) of head problem h, used to derive its seed."""
        if self.unit_kind == "doc":
            return 0, h // self.heads_per_unit, h % self.heads_per_unit
        if self.unit_kind == "layer":
            return h // self.heads_per_unit, 0, h % self.heads_per_unit
        return 0, 0, h


WORKLOADS = [
    # single head, fp32, d=64, T=n=1024, t=64 (16x)
    Workload("single_head_f32_T1k", heads=1, d=64, T=1024, n=1024, t=64, dtype="f32",
             causal=False, group=1),
    # 64 documents x 8 KV heads, T=n=2048, t=64 (32x)
    Workload("docs64x8_T2k", heads=512, d=128, T=2048, n=2048, t=64, dtype="bf16",
             causal=False, group=1, unit_kind="doc"),
    # 36 layers x 8 KV heads, T=4096, GQA 4 -> n=16384, t=128 (32x)
    Workload("layers36x8_T4k_gqa4", heads=288, d=128, T=4096, n=16384, t=128, dtype="bf16",
             causal=False, group=4, unit_kind="layer"),
    # one layer, 8 KV heads, T=32768, GQA 4 -> n=131072, causal, t=1024 (32x)
    Workload("causal8_T32k_gqa4", heads=8, d=128, T=32768, n=131072, t=1024, dtype="bf16",
             causal=True, group=4),
    # one KV head, T=n=131072, t=4096 (32x), extra x4 needles
    Workload("single_head_T128k", heads=1, d=128, T=131072, n=131072, t=4096, dtype="bf16",
             causal=False, group=1, extra_needles=True),
]

BY_NAME = {w.name: w for w in WORKLOADS}


def small_variant(w: Workload, *, heads: int | None = None, T: int | None = None,
                  t: int | None = None, name_suffix: str = "_small") -> Workload:
    """Same generator and structure at a reduced size (for oracle-speed parity cases)."""
    import dataclasses
    T2 = T if T is not None else w.T
    n2 = w.group * T2 if (w.causal or w.group > 1) else (T2 if w.n == w.T else w.n)
    return dataclasses.replace(w, name=w.name + name_suffix, heads=heads or w.heads, T=T2, n=n2,
                               t=t if t is not None else max(1, T2 // (w.T // w.t)))
