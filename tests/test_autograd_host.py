"""Host-side checks of the autograd wrapper (no GPU): it exists, it refuses
CPU tensors instead of computing anything on the host, and its "auto"
backward schedule is the recomputing one."""
import pytest
import torch

import workloads as W

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")


def test_exported():
    assert callable(bsr.block_sparse_attention)
    assert "block_sparse_attention" in bsr.__all__


def test_cpu_tensors_rejected():
    bm = W.block_mask("local", 2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    q = torch.randn(1, 1, 256, 64, requires_grad=True)
    with pytest.raises(ValueError, match="GPU"):
        bsr.block_sparse_attention(q, q, q, s)


def test_unknown_backward_schedule_rejected():
    bm = W.block_mask("local", 2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    q = torch.randn(1, 1, 256, 64, requires_grad=True)
    with pytest.raises(ValueError, match="backward_schedule"):
        bsr.block_sparse_attention(q, q, q, s, backward_schedule="fastest")


def test_auto_backward_schedule_choice():
    """"auto" recomputes the scores in both backward passes for every dtype
    and head dim (the faster schedule on the measured workloads)."""
    pick = bsr.autograd.backward_schedule_for
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        for d in (16, 64, 128, 144, 192, 256, 272, 512):
            assert pick(dt, d) == "recompute"
