"""The five seeded workloads the decode step is measured and checked on.

Shapes: B sequences, blocks of L positions, hidden size H, vocabulary V.
The pages give no shapes; these are 8B-class stand-ins (hidden 2048, vocab
126464 / 157184) plus a tiny float32 case.  Policies follow the three
strategies of the dInfer explainer page ("decoding strategy component":
threshold, hierarchical and credit decoding).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

THRESHOLD, HIERARCHICAL, CREDIT = 0, 1, 2


@dataclass(frozen=True)
class SeqPolicy:
    kind: int
    threshold: float          # tau (threshold / hierarchical) or theta (credit)
    decay: float = 0.0        # credit only
    max_depth: int = 0        # hierarchical only; 0 = unbounded


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    L: int
    H: int
    V: int
    dtype: str                      # "f32" or "bf16"
    policies: List[SeqPolicy]
    a_max: float
    seeds: List[int]
    redraw_p: List[float]           # per sequence planted-token re-draw probability
    blocks: int                     # blocks per sequence in a full run
    steps: int = 0                  # fixed step count (0 = until the blocks are done)
    note: str = field(default="")

    @property
    def M(self) -> int:
        return self.B * self.L


def _thr(t=0.9):
    return SeqPolicy(THRESHOLD, t)


def _credit():
    return SeqPolicy(CREDIT, 1.2, 0.7)


def _hier(t=0.7):
    return SeqPolicy(HIERARCHICAL, t)


WORKLOADS = {
    "tiny_threshold_f32": Workload(
        "tiny_threshold_f32", 1, 8, 64, 1024, "f32", [_thr()], 40.0, [0], [0.0], 1,
        note="B=1, L=8, H=64, V=1024, float32, threshold 0.9, one block"),
    "threshold_b1_l32": Workload(
        "threshold_b1_l32", 1, 32, 2048, 126464, "bf16", [_thr()], 60.0, [0], [0.0], 32,
        note="B=1, L=32, H=2048, V=126464, bf16, threshold 0.9, 32 blocks"),
    "credit_b1_l32": Workload(
        "credit_b1_l32", 1, 32, 2048, 126464, "bf16", [_credit()], 60.0, [0], [0.3], 32,
        note="B=1, L=32, H=2048, V=126464, bf16, credit (decay 0.7, bar 1.2, 4 slots), re-draw 0.3"),
    "hierarchical_b1_l64": Workload(
        "hierarchical_b1_l64", 1, 64, 2048, 126464, "bf16", [_hier()], 60.0, [0], [0.0], 32,
        note="B=1, L=64, H=2048, V=126464, bf16, hierarchical 0.7, 32 blocks"),
    "mixed_b16_l32": Workload(
        "mixed_b16_l32", 16, 32, 2048, 157184, "bf16",
        [_thr()] * 8 + [_credit()] * 8, 60.0, list(range(16)), [0.0] * 8 + [0.3] * 8, 0,
        steps=64,
        note="B=16, L=32 (512 rows), H=2048, V=157184, bf16; sequences 0-7 threshold 0.9, 8-15 credit"),
}

ORDER = ["tiny_threshold_f32", "threshold_b1_l32", "credit_b1_l32", "hierarchical_b1_l64", "mixed_b16_l32"]
