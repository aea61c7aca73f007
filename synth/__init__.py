"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method (no quantisation, no GEMM):
only random draws of the fp32 source matrices, the expert index vector of the
contiguous layout and the per-expert row counts of the masked layout, plus the
workload shapes.  Both the CPU oracle and the HIP library consume what it
produces; neither is imported here.

Recipe (the pages name DeepSeek-V3/R1 inference shapes for their dense
benchmark, GeekNews topic 19444, "Performans degerlendirmesi", but list no
sizes; the sizes below are the workloads this library is measured on):

* a ``torch.Generator('cpu')`` seeded per problem; A [M, K] is drawn first,
  then B, both N(0, 1) in float32;
* contiguous layout: expert e owns ``rows[e]`` consecutive rows; each segment
  is padded up to a multiple of 128 rows with index -1 (``pad_to``);
* masked layout: per-expert valid counts drawn uniformly from 0..M_cap by a
  second generator with the same seed.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

ALIGN = 128


def normal(shape, gen: torch.Generator) -> torch.Tensor:
    """float32 N(0,1) on the CPU from ``gen``."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32)


def dense_problem(M: int, N: int, K: int, seed: int = 0):
    """fp32 A [M,K], B [N,K] (CPU tensors), A drawn first."""
    g = torch.Generator("cpu").manual_seed(seed)
    A = normal((M, K), g)
    B = normal((N, K), g)
    return A, B


def contiguous_indices(rows_per_expert, pad_to: int = ALIGN) -> np.ndarray:
    """int32 per-row expert index, sorted ascending, each segment padded to ``pad_to`` with -1."""
    out = []
    for e, r in enumerate(rows_per_expert):
        padded = -(-int(r) // pad_to) * pad_to
        out.append(np.full(int(r), e, np.int32))
        out.append(np.full(padded - int(r), -1, np.int32))
    return np.concatenate(out) if out else np.zeros(0, np.int32)


def contiguous_problem(rows_per_expert, N: int, K: int, seed: int = 0, pad_to: int = ALIGN):
    """fp32 A [M_total,K], B [G,N,K] and the int32 index vector (M_total padded)."""
    idx = contiguous_indices(rows_per_expert, pad_to)
    G = len(rows_per_expert)
    g = torch.Generator("cpu").manual_seed(seed)
    A = normal((idx.shape[0], K), g)
    B = normal((G, N, K), g)
    return A, B, idx


def masked_counts(G: int, M_cap: int, seed: int = 0) -> np.ndarray:
    """int32 [G] valid-row counts, uniform over 0..M_cap."""
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(0, M_cap + 1, (G,), generator=g).numpy().astype(np.int32)


def masked_problem(G: int, M_cap: int, N: int, K: int, seed: int = 0):
    """fp32 A [G,M_cap,K] (rows past the count are drawn too), B [G,N,K], counts [G]."""
    g = torch.Generator("cpu").manual_seed(seed)
    A = normal((G, M_cap, K), g)
    B = normal((G, N, K), g)
    return A, B, masked_counts(G, M_cap, seed)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "dense" | "contiguous" | "masked"
    shapes: tuple = field(default_factory=tuple)  # dense: (M,N,K); contiguous: (G,rows,N,K); masked: (G,M_cap,N,K)


#: Small dense case the oracle finishes in well under a second.
SMALL_DENSE = Workload("dense_small", "dense", ((128, 256, 512),))
#: Dense inference GEMMs at M=4096.
DENSE_M4096 = Workload(
    "dense_m4096",
    "dense",
    ((4096, 2112, 7168), (4096, 24576, 1536), (4096, 7168, 16384), (4096, 4096, 7168), (4096, 7168, 2048)),
)
#: Small-M decode GEMMs (HBM-bound).
DENSE_SMALL_M = Workload(
    "dense_small_m",
    "dense",
    tuple((m, n, k) for m in (64, 128) for (n, k) in ((2112, 7168), (4096, 7168), (7168, 2048))),
)
#: Contiguous MoE: 8 experts x 4096 rows, N=4096, K=7168.
CONTIGUOUS_8x4096 = Workload("contiguous_8x4096", "contiguous", ((8, 4096, 4096, 7168),))
#: Masked MoE decode: 16 experts, capacity 256.
MASKED_16x256 = Workload("masked_16x256", "masked", ((16, 256, 4096, 7168), (16, 256, 7168, 2048)))

WORKLOADS = {w.name: w for w in (SMALL_DENSE, DENSE_M4096, DENSE_SMALL_M, CONTIGUOUS_8x4096, MASKED_16x256)}
