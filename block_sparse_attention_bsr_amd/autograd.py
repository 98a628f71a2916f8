"""PyTorch autograd over the C ABI: block-sparse attention as registered ops.

Two operators, defined and implemented in C++ (``csrc/torch_ops.cpp``, built
in-tree as ``libbsr_attn_torch.so``), wrap the library's entry points:

    bsr_attn::attention_fwd(q, k, v, structure_id, scale, backward_schedule)
        -> (O, row_max, row_denom)                       (bsr_attn_fwd)
    bsr_attn::attention_bwd(q, k, v, o, d_o, row_max, row_denom,
                            structure_id, scale, backward_schedule)
        -> (dQ, dK, dV)                   (bsr_attn_bwd or bsr_attn_bwd_ds)

The forward operator's autograd kernel is registered on the operator (page
"trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: autograd on the native path is
registered on the ops rather than written as a Python autograd.Function). It
saves (Q, K, V, O, row_max, row_denom) and calls the backward operator with
those saved statistics instead of recomputing them (page "trnsparse 0.4.1 ->
0.6.0", CHANGELOG 0.5.1: the forward saves the six tensors and the backward
skips the statistics passes). Gradients flow through O only: the statistics
are non-differentiable. The backward operator refuses a second backward
instead of returning wrong second-order gradients.

This module registers the operators' shape functions (fake / meta kernels, so
they trace under torch.compile and fake tensors); the real kernels exist for
GPU tensors only, and every step runs in the library's HIP kernels. Operators
cannot take a Python object, so a Structure is passed by a process-local
integer id (``_structure_id``), under which its handle and its device plans
are registered with the operator library while the structure is alive.
"""
from __future__ import annotations

import ctypes
import itertools
import math
import weakref
from pathlib import Path

import torch

from . import Structure, _destroy_hooks

__all__ = ["block_sparse_attention", "attention_fwd", "attention_bwd", "TORCH_LIBRARY_PATH"]

TORCH_LIBRARY_PATH = Path(__file__).resolve().parent / "libbsr_attn_torch.so"
_SCHEDULES = ("auto", "recompute", "store_ds")

_ops_lib = None


def _load_ops() -> ctypes.CDLL | None:
    """Load the operator library (once); None if it has not been built."""
    global _ops_lib
    if _ops_lib is None and TORCH_LIBRARY_PATH.exists():
        # It links libbsr_attn.so from its own directory: the file the binding
        # loads by default, so both use one copy of the library.
        torch.ops.load_library(str(TORCH_LIBRARY_PATH))
        L = ctypes.CDLL(str(TORCH_LIBRARY_PATH))
        L.bsr_attn_torch_register.argtypes = [ctypes.c_int64, ctypes.c_void_p]
        L.bsr_attn_torch_register.restype = ctypes.c_int
        L.bsr_attn_torch_register_plan.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        L.bsr_attn_torch_register_plan.restype = ctypes.c_int
        L.bsr_attn_torch_unregister.argtypes = [ctypes.c_int64]
        L.bsr_attn_torch_unregister.restype = None
        _ops_lib = L
    return _ops_lib


def _ops() -> ctypes.CDLL:
    L = _load_ops()
    if L is None:
        raise RuntimeError(f"{TORCH_LIBRARY_PATH} is missing: build it with "
                           "`python -m block_sparse_attention_bsr_amd.build`")
    return L


_ids = itertools.count(1)
_structures: "weakref.WeakValueDictionary[int, Structure]" = weakref.WeakValueDictionary()


def _structure_id(s: Structure, device: torch.device | None = None) -> int:
    """The structure's operator id, registered on first use; also registers
    its device plan for ``device`` (default: the current GPU, if any)."""
    sid = getattr(s, "_op_id", None)
    if sid is None:
        sid = next(_ids)
        if _ops().bsr_attn_torch_register(sid, s.handle) != 0:
            raise RuntimeError("registering the structure with the operator library failed")
        s._op_id = sid
        s._op_devices = set()
        _structures[sid] = s
    if device is None and torch.cuda.is_available():
        device = torch.device("cuda", torch.cuda.current_device())
    if device is not None and device.type == "cuda":
        index = device.index if device.index is not None else torch.cuda.current_device()
        if index not in s._op_devices:
            plan = s.device_plan(torch.device("cuda", index))
            if _ops().bsr_attn_torch_register_plan(sid, index, plan.data_ptr()) != 0:
                raise RuntimeError("registering the device plan with the operator library failed")
            s._op_devices.add(index)
    return sid


def _forget(s: Structure) -> None:
    sid = getattr(s, "_op_id", None)
    if sid is not None and _ops_lib is not None:
        _ops_lib.bsr_attn_torch_unregister(sid)


_destroy_hooks.append(_forget)


def _structure(sid: int) -> Structure:
    s = _structures.get(sid)
    if s is None:
        raise ValueError(f"no live Structure with id {sid}")
    return s


attention_fwd = attention_bwd = None
if _load_ops() is not None:
    attention_fwd = torch.ops.bsr_attn.attention_fwd
    attention_bwd = torch.ops.bsr_attn.attention_bwd

    @torch.library.register_fake("bsr_attn::attention_fwd")
    def _attention_fwd_fake(q, k, v, structure_id, scale, backward_schedule):
        stats = q.new_empty(q.shape[:3], dtype=torch.float32)
        return torch.empty_like(q), stats, torch.empty_like(stats)

    @torch.library.register_fake("bsr_attn::attention_bwd")
    def _attention_bwd_fake(q, k, v, o, d_o, row_max, row_denom, structure_id, scale, backward_schedule):
        return torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)


def block_sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, structure: Structure,
                           scale: float | None = None, return_stats: bool = False,
                           backward_schedule: str = "recompute"):
    """Softmax attention over the stored 128 x 128 blocks of ``structure``.

    q, k, v: [batch, heads, seq_len, head_dim] on one GPU, one dtype (fp32,
    bf16 or fp16); non-contiguous inputs are copied. ``scale`` defaults to
    1/sqrt(head_dim). Returns O, or (O, row_max, row_denom) with
    ``return_stats`` (fp32 [batch, heads, seq_len]; P = exp(S - row_max) /
    row_denom). Differentiable in q, k and v (once). ``backward_schedule``:
    "recompute" (``bsr_attn_bwd``: both backward passes recompute the scores;
    the default, and the faster schedule on every head_dim 128 workload
    measured) or "store_ds" (``bsr_attn_bwd_ds``, bf16/fp16: the dK/dV pass
    stores dS and dQ reads it; at head_dim 256 it measured about 3 % faster on
    the random 10 % workload, for an extra batch*heads*nnzb*32 KB of
    workspace). "auto" is accepted as "recompute".
    """
    if backward_schedule not in _SCHEDULES:
        raise ValueError(f"backward_schedule must be one of {sorted(_SCHEDULES)}")
    if backward_schedule == "auto":
        backward_schedule = "recompute"
    if q.device.type != "cuda":
        raise ValueError("operands must be on a GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    sid = _structure_id(structure, q.device)
    o, row_max, row_denom = torch.ops.bsr_attn.attention_fwd(q.contiguous(), k.contiguous(), v.contiguous(), sid,
                                                             float(scale), backward_schedule)
    return (o, row_max, row_denom) if return_stats else o
