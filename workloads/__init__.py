"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no attention arithmetic: only block-mask constructors, the
BSR encoding of a boolean block mask, and seeded random tensors. Both the HIP
path and the oracle consume exactly what it returns.

Mask kinds (nb = number of 128-blocks per side, i = block row, j = block column):

- ``local``    keep |i - j| <= 1 (window radius one block: three blocks per
               row). Page "trnsparse 0.7.0 -> 0.9.0",
               benchmarks/bench_native_trn2.py, attention masks.
- ``dilated_pages`` keep (j - i) divisible by 4 (stride-4 dilation, both
               sides, no band): the same page's dilated mask.
- ``dilated``  keep |i - j| <= 1, or (i - j) divisible by 4 with j <= i: the
               dilated mask of the 2048-token, 8-head benchmark configuration.
- ``global``   the local band plus all of block row 0 and block column 0
               (global tokens): the same page's global mask.
- ``random``   k = max(1, round(density * nb^2)) distinct blocks drawn by a
               seeded permutation of the nb^2 positions (the same page's
               random BSR recipe for its SpMM section), with the diagonal
               forced on so that every row and column attends to something.
- ``full``     every block (dense attention, the "full-attention edge case").
- ``diagonal`` only the diagonal blocks.

Tensors follow the page's attention data recipe: one torch generator seeded
once, Q, K, V, dO drawn in that order from N(0, 1), then rounded to the
operand dtype, so that both sides see values exactly representable in it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

BLOCK = 128

MASK_KINDS = ("local", "dilated_pages", "dilated", "global", "random", "full", "diagonal")


def block_mask(kind: str, nb: int, density: float | None = None, seed: int = 0) -> np.ndarray:
    """Boolean [nb, nb] block mask of the given kind."""
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    if kind == "local":
        m = np.abs(i - j) <= 1
    elif kind == "dilated_pages":
        m = (j - i) % 4 == 0
    elif kind == "dilated":
        m = (np.abs(i - j) <= 1) | (((i - j) % 4 == 0) & (j <= i))
    elif kind == "global":
        m = np.abs(i - j) <= 1
        m[0, :] = True
        m[:, 0] = True
    elif kind == "random":
        if density is None:
            raise ValueError("random mask needs a density")
        total = nb * nb
        k = max(1, round(density * total))
        g = torch.Generator().manual_seed(seed)
        flat = torch.randperm(total, generator=g)[:k].numpy()
        m = np.zeros((nb, nb), dtype=bool)
        m[flat // nb, flat % nb] = True
        m[np.arange(nb), np.arange(nb)] = True
    elif kind == "full":
        m = np.ones((nb, nb), dtype=bool)
    elif kind == "diagonal":
        m = np.eye(nb, dtype=bool)
    else:
        raise ValueError(f"unknown mask kind {kind!r}")
    return np.ascontiguousarray(m.astype(bool))


def bsr_from_block_mask(bm: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(row_ptr int32[nb+1], col_idx int32[nnzb]) of a boolean block mask,
    columns ascending within each row."""
    bm = np.asarray(bm, dtype=bool)
    counts = bm.sum(axis=1)
    row_ptr = np.zeros(bm.shape[0] + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(bm)[1].astype(np.int32)
    return row_ptr, col_idx


def block_mask_from_bsr(row_ptr, col_idx, nb: int) -> np.ndarray:
    m = np.zeros((nb, nb), dtype=bool)
    for r in range(nb):
        m[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return m


_TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def make_inputs(batch: int, heads: int, seq: int, head_dim: int, dtype: str = "fp32",
                seed: int = 0) -> tuple[torch.Tensor, ...]:
    """(Q, K, V, dO) as CPU fp32 tensors [B, H, S, D] holding values exactly
    representable in ``dtype``."""
    g = torch.Generator().manual_seed(seed)
    dt = _TORCH_DTYPES[dtype]
    shape = (batch, heads, seq, head_dim)
    out = []
    for _ in range(4):
        out.append(torch.randn(shape, generator=g).to(dt).float())
    return tuple(out)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# The benchmark configurations: (name, dtype, batch, heads, seq, head_dim, mask, density)
CONFIGS = {
    "c1_fp32_local": ("fp32", 1, 1, 512, 64, "local", None),
    "c2_bf16_dilated": ("bf16", 1, 8, 2048, 128, "dilated", None),
    "c3_bf16_global": ("bf16", 1, 16, 8192, 128, "global", None),
    "c4_bf16_rand10_d256": ("bf16", 1, 8, 8192, 256, "random", 0.10),
}
for _d in (0.01, 0.05, 0.10, 0.25, 0.50):
    for _dt in ("fp32", "bf16"):
        CONFIGS[f"c5_{_dt}_rand{int(round(_d * 100)):02d}"] = (_dt, 1, 8, 8192, 128, "random", _d)
# Not a benchmark configuration: the 10 % random workload with fp16 operands,
# a test case for the fp16 path.
CONFIGS["x_fp16_rand10"] = ("fp16", 1, 8, 8192, 128, "random", 0.10)
# Not a benchmark configuration either: head_dim 512 (the wide-head path) on
# the 10 % random workload.
CONFIGS["x_bf16_rand10_d512"] = ("bf16", 1, 8, 8192, 512, "random", 0.10)


def config_mask(name: str) -> np.ndarray:
    dt, b, h, s, d, kind, dens = CONFIGS[name]
    return block_mask(kind, s // BLOCK, density=dens, seed=0)
