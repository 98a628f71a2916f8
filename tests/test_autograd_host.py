"""Host-side checks of the autograd wrapper (no GPU): it exists, it refuses
CPU tensors instead of computing anything on the host, and its "auto"
backward schedule picks by dtype and head dim."""
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
    """"auto" stores dS for 16-bit operands at head dims 129..256 (the
    256-wide instances) and recomputes everywhere else."""
    pick = bsr.autograd.backward_schedule_for
    for dt in (torch.bfloat16, torch.float16):
        for d in (144, 192, 256):
            assert pick(dt, d) == "store_ds"
        for d in (16, 64, 128, 272, 512):
            assert pick(dt, d) == "recompute"
    for d in (64, 128, 256):
        assert pick(torch.float32, d) == "recompute"
