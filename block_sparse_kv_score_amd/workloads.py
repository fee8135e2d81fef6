"""The decode-step workloads, as named presets.

Shapes follow the model families the pages measure on (a Llama-3-8B-shaped
layer and a Llama-3.1-70B-shaped layer) and their context lengths; the data
itself is synthetic (see ``synth.py``).  Nothing in here computes anything.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

TABLE_FLAT = "flat"
TABLE_TWO_LEVEL = "two_level"
TABLE_PACKED_ROPE = "packed_rope"

#: appended tokens the generator prepares per (b, h): decode steps beyond
#: this many would need a larger capacity.
APPEND_CAPACITY = 256


@dataclass(frozen=True)
class Workload:
    wid: int                 # stable id, part of every seed
    name: str
    B: int                   # sequences
    Hq: int                  # query heads
    Hkv: int                 # KV heads (GQA group G = Hq / Hkv)
    D: int                   # head dim
    T0: int                  # context tokens present before step 1
    steps: int               # decode steps the workload specifies
    bs: int                  # block (= page) size in tokens
    ss: int                  # sub-block size in tokens
    k_e: int                 # eviction-part budget (blocks)
    k_q: int                 # query-part budget (blocks)
    splits: int              # split-K partitions of the selected list
    table: str = TABLE_FLAT
    append: bool = True      # each step appends one token per (b, h)
    select_all: bool = False  # skip scoring, attend over every block
    heavy_frac: float = 0.0  # share of key rows scaled up (heavy hitters)
    heavy_scale: float = 1.0
    e_sigma: float = 1.0     # std-dev of the eviction logits
    rope_base: float = 0.0
    n_docs: int = 0
    doc_len: int = 0
    prompt: int = 0          # prefill: the last `prompt` context tokens are the prompt
    seg_log2: int = 10       # two-level table: 1024-entry segments
    dir_entries: int = 256   # two-level table: directory size

    # -- derived -----------------------------------------------------------
    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def nsub(self) -> int:
        return self.bs // self.ss

    @property
    def n_append(self) -> int:
        return APPEND_CAPACITY if self.append else 0

    @property
    def max_blocks(self) -> int:
        """Logical block capacity per (b, h): context plus appended tokens."""
        return -(-(self.T0 + self.n_append) // self.bs)

    @property
    def blocks_log2(self) -> int:
        """Two-level table: per-(b, h) key space is 2^blocks_log2 blocks."""
        return max(self.seg_log2, math.ceil(math.log2(self.max_blocks)))

    @property
    def num_pages(self) -> int:
        return self.B * self.Hkv * self.max_blocks

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def k(self) -> int:
        return self.k_e + self.k_q

    def seq_len(self, step: int) -> int:
        """Tokens present during decode step ``step`` (1-based)."""
        return self.T0 + (step if self.append else 0)

    def scaled(self, **kw) -> "Workload":
        """Same workload family at other sizes (for parity tests)."""
        return replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        # 1: tiny NOSA decode, 16 steps
        Workload(1, "tiny_nosa", B=1, Hq=4, Hkv=1, D=64, T0=2048, steps=16,
                 bs=64, ss=16, k_e=4, k_q=4, splits=2),
        # 2: Llama-3-8B-shaped layer at 32K context (the headline workload)
        Workload(2, "llama3_8b_32k", B=32, Hq=32, Hkv=8, D=128, T0=32768, steps=8,
                 bs=64, ss=16, k_e=32, k_q=32, splits=1,
                 heavy_frac=0.01, heavy_scale=20.0, e_sigma=math.sqrt(2.0)),
        # 3: dense equivalence at the 8B shape, 8K context, every block
        Workload(3, "dense_8b_8k", B=32, Hq=32, Hkv=8, D=128, T0=8192, steps=1,
                 bs=64, ss=16, k_e=64, k_q=64, splits=16, append=False),
        # 4: Llama-3.1-70B-shaped layer at 256K context, two-level page table
        Workload(4, "llama31_70b_256k", B=8, Hq=64, Hkv=8, D=128, T0=262144, steps=4,
                 bs=128, ss=32, k_e=96, k_q=32, splits=4, table=TABLE_TWO_LEVEL),
        # 5: deferred RoPE over 8 documents of 4096 tokens, every block
        Workload(5, "lazy_rope_32k", B=64, Hq=32, Hkv=8, D=128, T0=32768, steps=1,
                 bs=64, ss=16, k_e=0, k_q=512, splits=1, table=TABLE_PACKED_ROPE,
                 append=False, select_all=True, rope_base=500000.0,
                 n_docs=8, doc_len=4096),
        # 6: the same deferred-RoPE cache with NOSA selection (64 of 512
        # blocks): query-aware scores with the per-document rotated query
        Workload(6, "lazy_rope_sparse_32k", B=64, Hq=32, Hkv=8, D=128, T0=32768, steps=4,
                 bs=64, ss=16, k_e=32, k_q=32, splits=1, table=TABLE_PACKED_ROPE,
                 append=False, rope_base=500000.0, n_docs=8, doc_len=4096),
        # 7: prefill over reused documents: 64 retrieved documents of 512
        # tokens, then a 512-token prompt (the last document) attending
        # causally over everything before it
        Workload(7, "lazy_prefill_33k", B=4, Hq=32, Hkv=8, D=128, T0=65 * 512, steps=1,
                 bs=64, ss=16, k_e=0, k_q=520, splits=1, table=TABLE_PACKED_ROPE,
                 append=False, select_all=True, rope_base=500000.0, n_docs=65, doc_len=512,
                 prompt=512),
    ]
}

HEADLINE = "llama3_8b_32k"
