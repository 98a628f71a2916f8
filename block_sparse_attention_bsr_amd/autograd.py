"""PyTorch autograd over the C ABI: a differentiable block-sparse attention.

The forward runs ``bsr_attn_fwd`` and saves (Q, K, V, O, row_max, row_denom);
the backward runs ``bsr_attn_bwd`` with those saved statistics instead of
recomputing them (page "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.1: the
forward saves the six tensors and the backward skips the statistics passes;
page "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: the composite attention op
carries the dQ / dK-dV backward). Gradients flow through O only: the returned
statistics are marked non-differentiable.

Every step runs in the library's kernels; on anything but a GPU tensor the
call raises, as the binding does.
"""
from __future__ import annotations

import torch

from . import Structure, bsr_attn_bwd, bsr_attn_bwd_ds, bsr_attn_fwd

_BACKWARDS = {"recompute": bsr_attn_bwd, "store_ds": bsr_attn_bwd_ds}
_SCHEDULES = ("auto",) + tuple(_BACKWARDS)


def backward_schedule_for(dtype: torch.dtype, head_dim: int) -> str:
    """The backward schedule "auto" picks: "recompute" for every dtype and
    head dim. With the score products' operand read-ahead the recomputing
    backward measured faster than storing dS at head_dim 256 too (random
    10 %, 8 x 8192 x 256: 0.288 vs 0.301 ms), as it already was on the
    global mask and at 1 % and 50 % density; storing dS kept a 3 % lead only
    on random 10 % at head_dim 128, too small a margin for a rule. fp32 has
    no dS-storing form, and at head_dim 512 both take the same path. The
    arguments are kept so that a rule can depend on them again."""
    del dtype, head_dim
    return "recompute"

__all__ = ["block_sparse_attention", "backward_schedule_for"]


class _BsrAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, structure: Structure, scale, backward_schedule):
        o, row_max, row_denom = bsr_attn_fwd(structure, q, k, v, scale)
        ctx.save_for_backward(q, k, v, o, row_max, row_denom)
        ctx.structure = structure
        ctx.scale = scale
        ctx.backward = _BACKWARDS[backward_schedule]
        ctx.mark_non_differentiable(row_max, row_denom)
        return o, row_max, row_denom

    @staticmethod
    def backward(ctx, d_o, _d_row_max, _d_row_denom):
        q, k, v, o, row_max, row_denom = ctx.saved_tensors
        if d_o is None:
            return None, None, None, None, None, None
        dq, dk, dv = ctx.backward(ctx.structure, q, k, v, o, d_o.contiguous(), row_max, row_denom, ctx.scale)
        return dq, dk, dv, None, None, None


def block_sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, structure: Structure,
                           scale: float | None = None, return_stats: bool = False,
                           backward_schedule: str = "auto"):
    """Softmax attention over the stored 128 x 128 blocks of ``structure``.

    q, k, v: [batch, heads, seq_len, head_dim] on one GPU, one dtype (fp32 or
    bf16); non-contiguous inputs are copied. ``scale`` defaults to
    1/sqrt(head_dim). Returns O, or (O, row_max, row_denom) with
    ``return_stats`` (fp32 [batch, heads, seq_len]; P = exp(S - row_max) /
    row_denom). Differentiable in q, k and v. ``backward_schedule``:
    "recompute" (``bsr_attn_bwd``: both backward passes recompute the scores),
    "store_ds" (``bsr_attn_bwd_ds``, bf16/fp16: the dK/dV pass stores dS
    and dQ reads it) or "auto" (``backward_schedule_for``: currently
    recompute everywhere).
    """
    if backward_schedule not in _SCHEDULES:
        raise ValueError(f"backward_schedule must be one of {sorted(_SCHEDULES)}")
    if backward_schedule == "auto":
        backward_schedule = backward_schedule_for(q.dtype, q.shape[-1])
    o, row_max, row_denom = _BsrAttention.apply(q.contiguous(), k.contiguous(), v.contiguous(), structure, scale,
                                                backward_schedule)
    return (o, row_max, row_denom) if return_stats else o
