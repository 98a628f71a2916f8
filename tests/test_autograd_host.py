"""Host-side checks of the autograd ops (no GPU): the registered custom ops
exist with fake kernels, the forward's registered backward calls the backward
op, a double backward raises, and CPU tensors are refused instead of being
computed on the host. Meta tensors run the fake kernels only."""
import pytest
import torch

import workloads as W

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")


def _structure():
    return bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 2)))


def test_exported():
    assert callable(bsr.block_sparse_attention)
    assert "block_sparse_attention" in bsr.__all__
    assert hasattr(torch.ops.bsr_attn, "attention_fwd") and hasattr(torch.ops.bsr_attn, "attention_bwd")


def test_cpu_tensors_rejected():
    s = _structure()
    q = torch.randn(1, 1, 256, 64, requires_grad=True)
    with pytest.raises(ValueError, match="GPU"):
        bsr.block_sparse_attention(q, q, q, s)
    # the op itself has no CPU kernel
    sid = bsr.autograd._structure_id(s)
    with pytest.raises(NotImplementedError):
        torch.ops.bsr_attn.attention_fwd(q.detach(), q.detach(), q.detach(), sid, 0.125, "recompute")


def test_unknown_backward_schedule_rejected():
    s = _structure()
    q = torch.randn(1, 1, 256, 64, requires_grad=True)
    with pytest.raises(ValueError, match="backward_schedule"):
        bsr.block_sparse_attention(q, q, q, s, backward_schedule="fastest")


def test_fake_kernels_and_registered_backward_on_meta():
    """Shapes and dtypes from the fake kernels; the statistics do not require
    grad; the gradient of O reaches q through the backward op."""
    s = _structure()
    sid = bsr.autograd._structure_id(s)
    q = torch.randn(2, 3, 256, 64, device="meta", dtype=torch.bfloat16, requires_grad=True)
    o, m, l_ = torch.ops.bsr_attn.attention_fwd(q, q, q, sid, 0.125, "recompute")
    assert o.shape == q.shape and o.dtype == torch.bfloat16
    assert m.shape == (2, 3, 256) and m.dtype == torch.float32 and l_.dtype == torch.float32
    assert o.requires_grad and not m.requires_grad and not l_.requires_grad
    (g,) = torch.autograd.grad(o, q, torch.empty_like(o))
    assert g.shape == q.shape and g.dtype == q.dtype


def test_double_backward_raises():
    """The backward op has no autograd formula: second-order gradients raise
    rather than come back silently wrong."""
    s = _structure()
    sid = bsr.autograd._structure_id(s)
    q = torch.randn(1, 1, 256, 64, device="meta", requires_grad=True)
    o, _, _ = torch.ops.bsr_attn.attention_fwd(q, q, q, sid, 0.125, "recompute")
    (g,) = torch.autograd.grad(o, q, torch.empty_like(o), create_graph=True)
    with pytest.raises(RuntimeError, match="no autograd formula"):
        g.sum().backward()


def test_dead_structure_id_raises():
    s = _structure()
    sid = bsr.autograd._structure_id(s)
    assert bsr.autograd._structure(sid) is s
    del s
    import gc
    gc.collect()
    with pytest.raises(ValueError, match="no live Structure"):
        bsr.autograd._structure(sid)


def test_operator_registry_threads():
    """The operator library's registry of live structures takes registrations
    and removals from many threads at once (the autograd engine runs the
    backward on a thread of its own) and ends empty of them."""
    import threading

    L = bsr.autograd._ops()
    s = _structure()
    errors = []

    def worker(base):
        for i in range(200):
            sid = 10_000_000 + base * 1000 + i
            if L.bsr_attn_torch_register(sid, s.handle) != 0:
                errors.append(("register", sid))
            if L.bsr_attn_torch_register_plan(sid, 0, 4096) != 0:
                errors.append(("plan", sid))
            L.bsr_attn_torch_unregister(sid)
            if L.bsr_attn_torch_register_plan(sid, 0, 4096) != 1:  # gone: refused
                errors.append(("stale", sid))

    threads = [threading.Thread(target=worker, args=(b,)) for b in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors
    # invalid arguments are refused
    assert L.bsr_attn_torch_register(1, None) == 1
    assert L.bsr_attn_torch_register(0, s.handle) == 1
