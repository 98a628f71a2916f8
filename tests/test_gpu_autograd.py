"""GPU: the autograd ops over the C ABI (registered torch.library custom ops).

Its gradients must be exactly the C ABI backward's (same kernels, same saved
statistics) for the loss <O, dO>, and must match the fp64 oracle within the
parity tolerance; a loss that is not linear in O (sum of O^2) must hand the
backward dO = 2 O; torch.library.opcheck must accept both ops (schema, fake
kernels against the real ones, autograd registration, AOT dispatch).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"fp32": 1e-4, "bf16": 2e-2}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("bf16", 128), ("bf16", 64)])
def test_autograd_matches_c_abi_and_oracle(dtype, D):
    bm = W.block_mask("global", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=2)
    q, k, v, do = W.make_inputs(1, 2, 512, D, dtype, seed=3)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    ql, kl, vl = (t.clone().requires_grad_() for t in (qd, kd, vd))
    o = bsr.block_sparse_attention(ql, kl, vl, s)
    o.backward(dod)
    # exactly the C ABI's results
    o2, m2, l2 = bsr.bsr_attn_fwd(s, qd, kd, vd)
    dq2, dk2, dv2 = bsr.bsr_attn_bwd(s, qd, kd, vd, o2, dod, m2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for g, ref in ((ql.grad, dq2), (kl.grad, dk2), (vl.grad, dv2)):
        assert torch.equal(g, ref)
    # and the oracle's
    qn, kn, vn, don = (t.double().numpy() for t in (q, k, v, do))  # already dtype-exact values
    o_r, _, _ = oracle.fwd(qn, kn, vn, rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(qn, kn, vn, don, rp, ci)
    assert rel(o.detach().float().cpu(), o_r) <= TOL[dtype]
    for g, ref in ((ql.grad, dq_r), (kl.grad, dk_r), (vl.grad, dv_r)):
        assert rel(g.float().cpu(), ref) <= TOL[dtype]


def test_autograd_nonlinear_loss_and_stats():
    bm = W.block_mask("local", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    q, k, v, _ = W.make_inputs(1, 1, 512, 64, "fp32", seed=5)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    ql, kl, vl = (t.clone().requires_grad_() for t in (qd, kd, vd))
    o, m, l_ = bsr.block_sparse_attention(ql, kl, vl, s, return_stats=True)
    assert not m.requires_grad and not l_.requires_grad
    (o * o).sum().backward()
    o2, m2, l2 = bsr.bsr_attn_fwd(s, qd, kd, vd)
    dq2, dk2, dv2 = bsr.bsr_attn_bwd(s, qd, kd, vd, o2, (2 * o2).contiguous(), m2, l2)
    torch.cuda.synchronize()
    assert torch.equal(m, m2) and torch.equal(l_, l2)
    for g, ref in ((ql.grad, dq2), (kl.grad, dk2), (vl.grad, dv2)):
        assert torch.equal(g, ref)


def test_autograd_noncontiguous_inputs():
    bm = W.block_mask("diagonal", 2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    dev = torch.device("cuda:0")
    base = torch.randn(1, 256, 2, 64, device=dev)  # [B, S, H, D] -> transpose to [B, H, S, D]
    q = base.transpose(1, 2).requires_grad_()
    assert not q.is_contiguous()
    o = bsr.block_sparse_attention(q, q, q, s)
    o.sum().backward()
    assert q.grad.shape == q.shape and torch.isfinite(q.grad).all()


def test_autograd_auto_schedule_head_dim_256():
    """The default ("auto") schedule at bf16 head_dim 256 is the recomputing
    backward: exactly bsr_attn_bwd's gradients, within tolerance of the
    oracle."""
    bm = W.block_mask("random", 4, density=0.5, seed=2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=2)
    q, k, v, do = W.make_inputs(1, 2, 512, 256, "bf16", seed=6)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, torch.bfloat16).contiguous() for t in (q, k, v, do))
    ql, kl, vl = (t.clone().requires_grad_() for t in (qd, kd, vd))
    bsr.block_sparse_attention(ql, kl, vl, s).backward(dod)
    o2, m2, l2 = bsr.bsr_attn_fwd(s, qd, kd, vd)
    ref = bsr.bsr_attn_bwd(s, qd, kd, vd, o2, dod, m2, l2)
    torch.cuda.synchronize()
    for g, r in zip((ql.grad, kl.grad, vl.grad), ref):
        assert torch.equal(g, r)
    qn, kn, vn, don = (t.double().numpy() for t in (q, k, v, do))
    for g, r in zip((ql.grad, kl.grad, vl.grad), oracle.bwd(qn, kn, vn, don, rp, ci)):
        assert rel(g.float().cpu(), r) <= TOL["bf16"]


def test_autograd_store_ds_schedule():
    """backward_schedule="store_ds" hands back exactly bsr_attn_bwd_ds's
    gradients, within tolerance of the oracle."""
    bm = W.block_mask("global", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=2)
    q, k, v, do = W.make_inputs(1, 2, 512, 128, "bf16", seed=5)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, torch.bfloat16).contiguous() for t in (q, k, v, do))
    ql, kl, vl = (t.clone().requires_grad_() for t in (qd, kd, vd))
    bsr.block_sparse_attention(ql, kl, vl, s, backward_schedule="store_ds").backward(dod)
    o2, m2, l2 = bsr.bsr_attn_fwd(s, qd, kd, vd)
    ref = bsr.bsr_attn_bwd_ds(s, qd, kd, vd, o2, dod, m2, l2)
    torch.cuda.synchronize()
    for g, r in zip((ql.grad, kl.grad, vl.grad), ref):
        assert torch.equal(g, r)
    qn, kn, vn, don = (t.double().numpy() for t in (q, k, v, do))
    for g, r in zip((ql.grad, kl.grad, vl.grad), oracle.bwd(qn, kn, vn, don, rp, ci)):
        assert rel(g.float().cpu(), r) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_opcheck(dtype, D):
    bm = W.block_mask("global", 3)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    sid = bsr.autograd._structure_id(s)
    q, k, v, do = W.make_inputs(1, 2, 384, D, dtype, seed=8)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    scale = 1.0 / np.sqrt(D)
    ql, kl, vl = (t.clone().requires_grad_() for t in (qd, kd, vd))
    torch.library.opcheck(torch.ops.bsr_attn.attention_fwd.default, (ql, kl, vl, sid, scale, "recompute"))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd, scale)
    torch.library.opcheck(torch.ops.bsr_attn.attention_bwd.default,
                          (qd, kd, vd, o, dod, m, l_, sid, scale, "recompute"))


def test_operator_errors():
    """The C++ operators check their operands and the structure id before
    anything is enqueued: a dead structure, mismatched dtypes or shapes, a
    strided operand and an unknown schedule raise ValueError."""
    bm = W.block_mask("local", 2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    sid = bsr.autograd._structure_id(s)
    dev = torch.device("cuda:0")
    q = torch.randn(1, 2, 256, 64, device=dev)
    op_f, op_b = torch.ops.bsr_attn.attention_fwd, torch.ops.bsr_attn.attention_bwd
    with pytest.raises(ValueError, match="must match q"):
        op_f(q, q.half(), q, sid, 0.125, "recompute")
    with pytest.raises(ValueError, match="must match q"):
        op_f(q, q[:, :, :128].contiguous(), q, sid, 0.125, "recompute")
    with pytest.raises(ValueError, match="contiguous"):
        op_f(q, q.transpose(2, 3).contiguous().transpose(2, 3), q, sid, 0.125, "recompute")
    o, m, l_ = op_f(q, q, q, sid, 0.125, "recompute")
    with pytest.raises(ValueError, match="backward_schedule"):
        op_b(q, q, q, o, o, m, l_, sid, 0.125, "fastest")
    with pytest.raises(ValueError, match="row_max"):
        op_b(q, q, q, o, o, m.double(), l_, sid, 0.125, "recompute")
    torch.cuda.synchronize()
    del s
    import gc
    gc.collect()
    with pytest.raises(ValueError, match="no live Structure"):
        op_f(q, q, q, sid, 0.125, "recompute")
