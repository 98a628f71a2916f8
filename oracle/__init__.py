"""Oracle for BSR block-sparse softmax attention (fp64, CPU).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product package never does.

A thin ctypes wrapper over ``bsr_attn_oracle.c`` (plain C, fp64, OpenMP over
independent rows / key blocks). Every function takes NumPy arrays shaped
``[B, H, S, D]`` (any float dtype; converted to float64) and the BSR block
structure ``(row_ptr, col_idx)`` of ``block``-sized tiles shared by all
(batch, head) pairs. What each entry point computes, and the pages it follows,
is documented in the C source.
"""
from __future__ import annotations

import ctypes
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "bsr_attn_oracle.c"
LIBRARY = _HERE / "liboracle_bsr_attn.so"

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def compile_oracle(source: Path = SOURCE, output: Path = LIBRARY, extra_flags=()) -> Path:
    """Build the oracle with gcc (-O2 -fopenmp). Returns the library path."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags,
           str(source), "-o", str(output), "-lm"]
    subprocess.run(cmd, check=True)
    return output


class Oracle:
    """One loaded oracle library (the committed one, or a test's variant)."""

    def __init__(self, path: Path | str = LIBRARY):
        path = Path(path)
        if not path.exists():
            raise FileNotFoundError(f"oracle library not built: {path}")
        self.lib = ctypes.CDLL(str(path))
        head = [_i64, _i64, _i64, _i64, _i64, _p, _p, _dbl]
        L = self.lib
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_fwd.argtypes = head + [_p] * 6
        L.oracle_fwd_rows.argtypes = head + [_p] * 3 + [_i64, _p] + [_p] * 3
        L.oracle_bwd.argtypes = head + [_p] * 7
        L.oracle_bwd_rows.argtypes = head + [_p] * 4 + [_i64, _p, _p]
        L.oracle_bwd_cols.argtypes = head + [_p] * 4 + [_i64, _p, _p, _p]
        L.oracle_spmm.argtypes = [_i64, _i64, _i64, _p, _p, _p, _p, _p]
        L.oracle_spmm.restype = None
        for f in (L.oracle_fwd, L.oracle_fwd_rows, L.oracle_bwd, L.oracle_bwd_rows, L.oracle_bwd_cols):
            f.restype = None

    def threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    # -- argument marshalling -------------------------------------------------
    @staticmethod
    def _dense(x):
        return np.ascontiguousarray(np.asarray(x, dtype=np.float64))

    @staticmethod
    def _struct(row_ptr, col_idx):
        rp = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int32))
        ci = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int32))
        if ci.size == 0:
            ci = np.zeros(1, dtype=np.int32)  # a valid pointer; never read
        return rp, ci

    def _head(self, q, row_ptr, block, scale):
        B, H, S, D = q.shape
        nb = len(row_ptr) - 1
        if S != nb * block:
            raise ValueError(f"seq {S} != {nb} block rows x {block}")
        if scale is None:
            scale = 1.0 / np.sqrt(D)
        return B * H, S, D, nb, float(scale)

    # -- entry points ---------------------------------------------------------
    def fwd(self, q, k, v, row_ptr, col_idx, scale=None, block=128):
        """Returns (O [B,H,S,D], row_max [B,H,S], row_denom [B,H,S]) in fp64."""
        q, k, v = self._dense(q), self._dense(k), self._dense(v)
        rp, ci = self._struct(row_ptr, col_idx)
        BH, S, D, nb, scale = self._head(q, rp, block, scale)
        o = np.empty_like(q)
        m = np.empty(q.shape[:3])
        l_ = np.empty(q.shape[:3])
        self.lib.oracle_fwd(BH, S, D, block, nb, rp.ctypes.data, ci.ctypes.data, scale,
                            q.ctypes.data, k.ctypes.data, v.ctypes.data,
                            o.ctypes.data, m.ctypes.data, l_.ctypes.data)
        return o, m, l_

    def fwd_rows(self, q, k, v, row_ptr, col_idx, rows, scale=None, block=128):
        """Forward for flat rows ``bh * S + r`` only: (O [n,D], row_max [n], row_denom [n])."""
        q, k, v = self._dense(q), self._dense(k), self._dense(v)
        rp, ci = self._struct(row_ptr, col_idx)
        BH, S, D, nb, scale = self._head(q, rp, block, scale)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows)
        o = np.empty((n, D))
        m = np.empty(n)
        l_ = np.empty(n)
        self.lib.oracle_fwd_rows(BH, S, D, block, nb, rp.ctypes.data, ci.ctypes.data, scale,
                                 q.ctypes.data, k.ctypes.data, v.ctypes.data, n, rows.ctypes.data,
                                 o.ctypes.data, m.ctypes.data, l_.ctypes.data)
        return o, m, l_

    def bwd(self, q, k, v, dout, row_ptr, col_idx, scale=None, block=128):
        """Returns (dQ, dK, dV), each [B,H,S,D] fp64, for the loss <O, dout>."""
        q, k, v, dout = self._dense(q), self._dense(k), self._dense(v), self._dense(dout)
        rp, ci = self._struct(row_ptr, col_idx)
        BH, S, D, nb, scale = self._head(q, rp, block, scale)
        dq, dk, dv = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        self.lib.oracle_bwd(BH, S, D, block, nb, rp.ctypes.data, ci.ctypes.data, scale,
                            q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                            dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
        return dq, dk, dv

    def bwd_rows(self, q, k, v, dout, row_ptr, col_idx, rows, scale=None, block=128):
        """dQ for flat query rows ``bh * S + r``: [n, D]."""
        q, k, v, dout = self._dense(q), self._dense(k), self._dense(v), self._dense(dout)
        rp, ci = self._struct(row_ptr, col_idx)
        BH, S, D, nb, scale = self._head(q, rp, block, scale)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        dq = np.empty((len(rows), D))
        self.lib.oracle_bwd_rows(BH, S, D, block, nb, rp.ctypes.data, ci.ctypes.data, scale,
                                 q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                 len(rows), rows.ctypes.data, dq.ctypes.data)
        return dq

    def bwd_cols(self, q, k, v, dout, row_ptr, col_idx, cols, scale=None, block=128):
        """(dK [n,D], dV [n,D]) for flat keys ``bh * S + c``."""
        q, k, v, dout = self._dense(q), self._dense(k), self._dense(v), self._dense(dout)
        rp, ci = self._struct(row_ptr, col_idx)
        BH, S, D, nb, scale = self._head(q, rp, block, scale)
        cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        dk = np.empty((len(cols), D))
        dv = np.empty((len(cols), D))
        self.lib.oracle_bwd_cols(BH, S, D, block, nb, rp.ctypes.data, ci.ctypes.data, scale,
                                 q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                 len(cols), cols.ctypes.data, dk.ctypes.data, dv.ctypes.data)
        return dk, dv

    def spmm(self, blocks, b_dense, row_ptr, col_idx, block=128):
        """C = A B for A given by its stored blocks [nnzb, block, block] (BSR
        order) and B [nb*block, n]; returns C [nb*block, n] in fp64."""
        nnzb = len(np.asarray(col_idx))
        rp, ci = self._struct(row_ptr, col_idx)
        nb = len(rp) - 1
        blocks = np.ascontiguousarray(blocks, dtype=np.float64)
        if nnzb == 0:
            blocks = np.zeros((1, block, block))  # a valid pointer; never read
        bd = np.ascontiguousarray(b_dense, dtype=np.float64)
        if (nnzb and blocks.shape != (nnzb, block, block)) or bd.ndim != 2 or bd.shape[0] != nb * block:
            raise ValueError("blocks must be [nnzb, block, block] and B [nb*block, n]")
        c = np.empty((nb * block, bd.shape[1]))
        self.lib.oracle_spmm(nb, block, bd.shape[1], rp.ctypes.data, ci.ctypes.data, blocks.ctypes.data,
                             bd.ctypes.data, c.ctypes.data)
        return c


_default: Oracle | None = None


def default() -> Oracle:
    """The committed oracle, compiled on first use if no build is present."""
    global _default
    if _default is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            compile_oracle()
        _default = Oracle(LIBRARY)
    return _default


def fwd(*a, **kw):
    return default().fwd(*a, **kw)


def fwd_rows(*a, **kw):
    return default().fwd_rows(*a, **kw)


def bwd(*a, **kw):
    return default().bwd(*a, **kw)


def bwd_rows(*a, **kw):
    return default().bwd_rows(*a, **kw)


def bwd_cols(*a, **kw):
    return default().bwd_cols(*a, **kw)


def spmm(*a, **kw):
    return default().spmm(*a, **kw)


def threads() -> int:
    return default().threads()

