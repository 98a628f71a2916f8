"""PyTorch autograd over the C ABI: block-sparse attention as registered ops.

Two ``torch.library`` custom ops wrap the library's entry points:

    bsr_attn::attention_fwd(q, k, v, structure_id, scale, backward_schedule)
        -> (O, row_max, row_denom)                       (bsr_attn_fwd)
    bsr_attn::attention_bwd(q, k, v, o, d_o, row_max, row_denom,
                            structure_id, scale, backward_schedule)
        -> (dQ, dK, dV)                   (bsr_attn_bwd or bsr_attn_bwd_ds)

The forward op's backward is registered with ``torch.library.register_autograd``
(page "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: autograd on the native path
is registered on the ops rather than written as an autograd.Function). It saves
(Q, K, V, O, row_max, row_denom) and calls the backward op with those saved
statistics instead of recomputing them (page "trnsparse 0.4.1 -> 0.6.0",
CHANGELOG 0.5.1: the forward saves the six tensors and the backward skips the
statistics passes). Gradients flow through O only: the statistics are marked
non-differentiable. The backward op itself has no autograd formula, so a
double backward raises instead of returning wrong second-order gradients.

Both ops have fake (meta) kernels, so they trace under torch.compile / fake
tensors; their real kernels are registered for GPU tensors only, and every
step runs in the library's HIP kernels. Custom ops cannot take a Python
object, so a Structure is passed by a process-local integer id
(``Structure.op_id``), looked up while the structure is alive.
"""
from __future__ import annotations

import itertools
import math
import weakref

import torch

from . import Structure, bsr_attn_bwd, bsr_attn_bwd_ds, bsr_attn_fwd

__all__ = ["block_sparse_attention", "attention_fwd", "attention_bwd"]

_BACKWARDS = {"recompute": bsr_attn_bwd, "store_ds": bsr_attn_bwd_ds}
_SCHEDULES = ("auto",) + tuple(_BACKWARDS)

_ids = itertools.count(1)
_structures: "weakref.WeakValueDictionary[int, Structure]" = weakref.WeakValueDictionary()


def _structure_id(s: Structure) -> int:
    sid = getattr(s, "_op_id", None)
    if sid is None:
        sid = next(_ids)
        s._op_id = sid
        _structures[sid] = s
    return sid


def _structure(sid: int) -> Structure:
    s = _structures.get(sid)
    if s is None:
        raise ValueError(f"no live Structure with id {sid}")
    return s


@torch.library.custom_op("bsr_attn::attention_fwd", mutates_args=(), device_types="cuda")
def attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, structure_id: int, scale: float,
                  backward_schedule: str) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    return bsr_attn_fwd(_structure(structure_id), q, k, v, scale)


@attention_fwd.register_fake
def _attention_fwd_fake(q, k, v, structure_id, scale, backward_schedule):
    stats = q.new_empty(q.shape[:3], dtype=torch.float32)
    return torch.empty_like(q), stats, torch.empty_like(stats)


@torch.library.custom_op("bsr_attn::attention_bwd", mutates_args=(), device_types="cuda")
def attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, d_o: torch.Tensor,
                  row_max: torch.Tensor, row_denom: torch.Tensor, structure_id: int, scale: float,
                  backward_schedule: str) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    return _BACKWARDS[backward_schedule](_structure(structure_id), q, k, v, o, d_o, row_max, row_denom, scale)


@attention_bwd.register_fake
def _attention_bwd_fake(q, k, v, o, d_o, row_max, row_denom, structure_id, scale, backward_schedule):
    return torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)


def _setup_context(ctx, inputs, output):
    q, k, v, structure_id, scale, backward_schedule = inputs
    o, row_max, row_denom = output
    ctx.save_for_backward(q, k, v, o, row_max, row_denom)
    ctx.structure_id = structure_id
    ctx.scale = scale
    ctx.backward_schedule = backward_schedule
    ctx.mark_non_differentiable(row_max, row_denom)


def _backward(ctx, d_o, _d_row_max, _d_row_denom):
    if d_o is None:
        return None, None, None, None, None, None
    q, k, v, o, row_max, row_denom = ctx.saved_tensors
    dq, dk, dv = attention_bwd(q, k, v, o, d_o.contiguous(), row_max, row_denom, ctx.structure_id, ctx.scale,
                               ctx.backward_schedule)
    return dq, dk, dv, None, None, None


torch.library.register_autograd("bsr_attn::attention_fwd", _backward, setup_context=_setup_context)


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
    the faster schedule on every measured workload, and the default) or
    "store_ds" (``bsr_attn_bwd_ds``, bf16/fp16: the dK/dV pass stores dS and
    dQ reads it). "auto" is accepted as "recompute".
    """
    if backward_schedule not in _SCHEDULES:
        raise ValueError(f"backward_schedule must be one of {sorted(_SCHEDULES)}")
    if backward_schedule == "auto":
        backward_schedule = "recompute"
    if q.device.type != "cuda":
        raise ValueError("operands must be on a GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    o, row_max, row_denom = attention_fwd(q.contiguous(), k.contiguous(), v.contiguous(), _structure_id(structure),
                                          float(scale), backward_schedule)
    return (o, row_max, row_denom) if return_stats else o
