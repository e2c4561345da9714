"""The synthetic workloads: shapes of the models the pages name, sizes of one CP rank's share.

Shapes only; there are no weights or datasets.  Each entry names the full-sequence problem
(B, S, Hq, Hkv, D), the simulated context-parallel degree and layout, which rank views are
run, and whether the backward is part of the workload.  Seeds are 1000 + workload number.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    cp: int
    layout: str         # "contiguous" or "zigzag"
    ranks: tuple
    backward: bool
    seed: int

    @property
    def chunk_rows(self) -> int:
        """Rows of one rank's slice (S / cp)."""
        return self.seq_len // self.cp

    @property
    def pair_rows(self) -> int:
        """L: rows of one pair block (a chunk for contiguous, a half-chunk for zigzag)."""
        return self.chunk_rows if self.layout == "contiguous" else self.chunk_rows // 2


WORKLOADS = {
    "tiny-f32-cp2": Workload("tiny-f32-cp2", 1, 256, 2, 2, 64, "f32", 2, "contiguous",
                             (0,), False, 1001),
    "gpt2s-bf16-cp4": Workload("gpt2s-bf16-cp4", 2, 4096, 12, 12, 64, "bf16", 4, "contiguous",
                               (0, 1, 2, 3), False, 1002),
    "llama-gqa-cp8-zigzag": Workload("llama-gqa-cp8-zigzag", 1, 32768, 32, 8, 128, "bf16", 8,
                                     "zigzag", (0, 7), True, 1003),
    "qwen3-ulysses-share": Workload("qwen3-ulysses-share", 1, 65536, 4, 1, 128, "bf16", 1,
                                    "contiguous", (0,), True, 1004),
    "long-ring-cp16-zigzag": Workload("long-ring-cp16-zigzag", 1, 262144, 16, 8, 128, "bf16", 16,
                                      "zigzag", (0, 15), True, 1005),
    "long-ring-cp16-contiguous": Workload("long-ring-cp16-contiguous", 1, 262144, 16, 8, 128, "bf16",
                                          16, "contiguous", (0, 15), True, 1005),
}
