"""Seeded synthetic workloads for the FP8 block-scaled GEMM and its MoE variants.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic: no E4M3 coding, no scale computation, no GEMM and no
output rounding.  Both the CPU oracle (tests) and the GPU path (tests, bench)
take their inputs from here, so the same bytes reach both sides.

Workloads (sizes as the workload list of the method states them):

* ``dense``      -- one M x N x K problem: A fp32 [M, K] drawn N(0, 1) with each
  row multiplied by 2**u, u ~ U[-4, 4] (log-uniform factor in [2^-4, 2^4]),
  and B fp32 [N, K] drawn N(0, 1).
* ``contiguous`` -- G experts, per-expert token counts drawn from a multinomial,
  each expert segment padded up to a multiple of 128 rows; ``m_indices`` holds
  the expert of every row and -1 on padding rows; padding rows of A are zero.
* ``masked``     -- G groups of ``max_m`` rows; ``masked_m[g]`` uniform on the
  integers 0..max_m.

Random streams: ``numpy.random.Generator(PCG64)`` seeded from
``numpy.random.SeedSequence(seed)``; child 0 drives routing and A, child
1 + g drives B of group g, so every group can be drawn on its own.  Large
tensors can instead be drawn on the GPU with a seeded ``torch.Generator``
(``draw_activation_device`` / ``draw_weight_device``): same distributions,
torch's own stream.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

SEGMENT_ALIGN = 128  # expert segments of the contiguous layout are padded to this

# (N, K) pairs of the dense LLM-layer shapes, and the M values they are crossed with.
DENSE_NK: Tuple[Tuple[int, int], ...] = (
    (2112, 7168), (24576, 1536), (7168, 16384), (4096, 7168), (7168, 2048))
DENSE_M: Tuple[int, ...] = (64, 128, 4096)
GROUPED_NK: Tuple[Tuple[int, int], ...] = ((4096, 7168), (7168, 2048))


def seed_for(config: int, shape_index: int) -> int:
    return 1000 * config + shape_index


def _streams(seed: int, num_groups: int) -> Tuple[np.random.Generator, List[np.random.Generator]]:
    children = np.random.SeedSequence(seed).spawn(1 + num_groups)
    gens = [np.random.Generator(np.random.PCG64(c)) for c in children]
    return gens[0], gens[1:]


def draw_activation(gen: np.random.Generator, rows: int, k: int) -> np.ndarray:
    """fp32 [rows, k]: N(0,1) draws, row i scaled by fp32(2**u_i), u_i ~ U[-4, 4]."""
    a = gen.standard_normal((rows, k), dtype=np.float32)
    u = gen.uniform(-4.0, 4.0, size=rows)
    a *= np.exp2(u).astype(np.float32)[:, None]
    return a


def draw_weight(gen: np.random.Generator, n: int, k: int) -> np.ndarray:
    return gen.standard_normal((n, k), dtype=np.float32)


@dataclass
class Dense:
    m: int
    n: int
    k: int
    seed: int
    a: np.ndarray          # fp32 [m, k]
    b: np.ndarray          # fp32 [n, k]


def dense(m: int, n: int, k: int, seed: int) -> Dense:
    g0, gb = _streams(seed, 1)
    return Dense(m, n, k, seed, draw_activation(g0, m, k), draw_weight(gb[0], n, k))


@dataclass
class Contiguous:
    num_groups: int
    n: int
    k: int
    seed: int
    counts: np.ndarray       # int64 [G] tokens per expert
    m_indices: np.ndarray    # int32 [m_total], -1 on padding rows
    a: np.ndarray            # fp32 [m_total, k], zero on padding rows
    b: Optional[np.ndarray]  # fp32 [G, n, k] (None when drawn on the device)

    @property
    def m_total(self) -> int:
        return int(self.m_indices.shape[0])

    @property
    def m_useful(self) -> int:
        return int((self.m_indices >= 0).sum())


def layout_contiguous(counts: Sequence[int], align: int = SEGMENT_ALIGN) -> np.ndarray:
    """m_indices for expert segments padded to ``align`` rows (-1 on padding)."""
    parts = []
    for g, c in enumerate(counts):
        c = int(c)
        padded = -(-c // align) * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:c] = g
        parts.append(seg)
    return np.concatenate(parts) if parts else np.zeros(0, np.int32)


def contiguous_routing(num_groups: int, tokens: int, probs: Sequence[float], seed: int):
    """(counts [G], m_indices [m_total]) of a contiguous workload, without drawing A or B."""
    g0, _ = _streams(seed, num_groups)
    counts = g0.multinomial(tokens, np.asarray(probs, dtype=np.float64))
    return counts, layout_contiguous(counts)


def contiguous(num_groups: int, tokens: int, probs: Sequence[float], n: int, k: int,
               seed: int, draw_b: bool = True) -> Contiguous:
    g0, gb = _streams(seed, num_groups)
    counts = g0.multinomial(tokens, np.asarray(probs, dtype=np.float64))
    m_indices = layout_contiguous(counts)
    valid = np.nonzero(m_indices >= 0)[0]
    a = np.zeros((m_indices.shape[0], k), dtype=np.float32)
    a[valid] = draw_activation(g0, valid.shape[0], k)
    b = np.stack([draw_weight(gb[g], n, k) for g in range(num_groups)]) if draw_b else None
    return Contiguous(num_groups, n, k, seed, counts, m_indices, a, b)


def draw_b_group_host(seed: int, num_groups: int, g: int, n: int, k: int) -> np.ndarray:
    """B of one group, from the same host stream ``contiguous`` uses for it."""
    _, gb = _streams(seed, num_groups)
    return draw_weight(gb[g], n, k)


def zipf_probs(num_experts: int, s: float) -> np.ndarray:
    """Expert popularity p(e) proportional to (e + 1)^-s, e = 0..num_experts-1."""
    w = (np.arange(num_experts, dtype=np.float64) + 1.0) ** (-s)
    return w / w.sum()


@dataclass
class Masked:
    num_groups: int
    max_m: int
    n: int
    k: int
    seed: int
    expected_m: int
    masked_m: np.ndarray     # int32 [G]
    a: np.ndarray            # fp32 [G, max_m, k]
    b: np.ndarray            # fp32 [G, n, k]

    @property
    def m_useful(self) -> int:
        return int(np.minimum(self.masked_m, self.max_m).sum())


def masked_counts(num_groups: int, max_m: int, seed: int) -> np.ndarray:
    """masked_m of a masked workload, without drawing A or B."""
    g0, _ = _streams(seed, num_groups)
    return g0.integers(0, max_m + 1, size=num_groups).astype(np.int32)


def masked(num_groups: int, max_m: int, n: int, k: int, seed: int,
           expected_m: int) -> Masked:
    g0, gb = _streams(seed, num_groups)
    masked_m = g0.integers(0, max_m + 1, size=num_groups).astype(np.int32)
    a = draw_activation(g0, num_groups * max_m, k).reshape(num_groups, max_m, k)
    b = np.stack([draw_weight(gb[g], n, k) for g in range(num_groups)])
    return Masked(num_groups, max_m, n, k, seed, expected_m, masked_m, a, b)


# ---------------------------------------------------------------- the five workloads

def config0() -> Dense:
    return dense(128, 256, 512, seed_for(0, 0))


def config1_shapes() -> List[Tuple[int, int, int]]:
    return [(m, n, k) for m in DENSE_M for (n, k) in DENSE_NK]


def config1(shape_index: int) -> Dense:
    m, n, k = config1_shapes()[shape_index]
    return dense(m, n, k, seed_for(1, shape_index))


def config2(shape_index: int) -> Contiguous:
    n, k = GROUPED_NK[shape_index]
    return contiguous(8, 8192, [1.0 / 8] * 8, n, k, seed_for(2, shape_index))


def config3(shape_index: int) -> Masked:
    n, k = GROUPED_NK[shape_index]
    return masked(16, 256, n, k, seed_for(3, shape_index), expected_m=128)


CONFIG4_EXPERTS = 256
CONFIG4_TOKENS = 32768
CONFIG4_ZIPF_S = 1.1
CONFIG4_NK = (4096, 7168)
CONFIG4_CAST_SHAPE = (32768, 7168)


def config2_routing(shape_index: int):
    return contiguous_routing(8, 8192, [1.0 / 8] * 8, seed_for(2, shape_index))


def config3_masked_m(shape_index: int) -> np.ndarray:
    return masked_counts(16, 256, seed_for(3, shape_index))


def config4_routing():
    return contiguous_routing(CONFIG4_EXPERTS, CONFIG4_TOKENS,
                              zipf_probs(CONFIG4_EXPERTS, CONFIG4_ZIPF_S), seed_for(4, 0))


def config4(draw_b: bool = False) -> Contiguous:
    """Zipf-routed contiguous MoE with power-of-two scales.  B (7.5 GB of codes at
    full size) is normally drawn per group on the device (``draw_weight_device``)."""
    n, k = CONFIG4_NK
    return contiguous(CONFIG4_EXPERTS, CONFIG4_TOKENS, zipf_probs(CONFIG4_EXPERTS, CONFIG4_ZIPF_S),
                      n, k, seed_for(4, 0), draw_b=draw_b)


def config4_cast_input(rows: Optional[int] = None):
    """bf16 activation [32768, 7168] for the per-token cast: drawn as the dense
    activation, stored as torch.bfloat16 (round-to-nearest-even storage)."""
    import torch
    r, k = CONFIG4_CAST_SHAPE
    r = r if rows is None else rows
    g0, _ = _streams(seed_for(4, 1), 0)
    return torch.from_numpy(draw_activation(g0, r, k)).to(torch.bfloat16)


# ---------------------------------------------------------------- device-side draws
# For full-size problems (hundreds of millions of values) the fp32 draws are made
# on the GPU by torch's seeded generator: same distributions as above, a
# different (torch) stream.  Stream ids keep A, row factors and each B group apart.

def _device_gen(seed: int, stream: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1_000_003 + stream) % (2 ** 63))
    return gen


def draw_activation_device(rows: int, k: int, seed: int, device, stream: int = 0):
    """fp32 [rows, k] on ``device``: N(0,1) times fp32(2**u) per row, u ~ U[-4, 4]."""
    import torch
    gen = _device_gen(seed, 2 * stream, device)
    a = torch.randn((rows, k), generator=gen, device=device, dtype=torch.float32)
    u = torch.rand((rows,), generator=_device_gen(seed, 2 * stream + 1, device), device=device,
                   dtype=torch.float64) * 8.0 - 4.0
    a *= torch.exp2(u).to(torch.float32)[:, None]
    return a


def draw_weight_device(n: int, k: int, seed: int, group: int, device):
    """fp32 [n, k] N(0,1) on ``device`` for group ``group``."""
    import torch
    gen = _device_gen(seed, 1_000_000 + group, device)
    return torch.randn((n, k), generator=gen, device=device, dtype=torch.float32)
