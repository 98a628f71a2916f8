"""Error measures shared by the parity tests (no attention arithmetic here).

rel        the pages' relative error of a whole tensor, ||x - ref|| / ||ref||
           in fp64 (Frobenius norm over every element), page
           "trnsparse 0.7.0 -> 0.9.0", benchmarks/bench_native_trn2.py,
           rel_err of the attention section.
row_err    the worst single row: for tensors of rows (the last axis is the
           row), max over rows r of ||x_r - ref_r|| / max(||ref_r||, rms),
           where rms is the root-mean-square row norm of ref. A row whose
           reference norm is at least the typical one is measured relative to
           itself; a row that is small only because its terms cancel is
           measured against the typical row norm, which is the scale its
           rounding errors have. For tensors of scalars per row (row_max,
           row_denom) the same with |.| per element.

A single wrong row among n rows moves `rel` by only about 1/sqrt(n) (0.003
at 131072 rows), below the bf16 gate; `row_err` reports it at about 1.
"""
from __future__ import annotations

import numpy as np


def rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def row_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape {x.shape} != {ref.shape}")
    if ref.size == 0:
        return 0.0
    if ref.ndim <= 1 or ref.shape[-1] == 1:
        d = np.abs(x - ref).reshape(-1)
        n = np.abs(ref).reshape(-1)
    else:
        d = np.linalg.norm((x - ref).reshape(-1, ref.shape[-1]), axis=1)
        n = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    rms = float(np.sqrt(np.mean(n * n)))
    if rms == 0.0:
        return float(d.max())
    return float(np.max(d / np.maximum(n, rms)))
