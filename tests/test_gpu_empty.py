"""Masks with no stored block at all, through every attention entry point.

Every query row is then an empty row (O = 0, row_max = -inf, row_denom = 0,
dQ = 0) and every key block is unreferenced (dK = dV = 0): the plain
definition's empty sums, which is also what the oracle returns. Outputs are
pre-filled with NaN and the C ABI is called directly, so the test sees that
every element is written, not left over from the allocator.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
pytestmark = pytest.mark.gpu
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsr.library()


def _nan_like(t, dtype=None, shape=None):
    return torch.full(shape if shape is not None else t.shape, float("nan"), dtype=dtype or t.dtype, device=t.device)


def _forward(entry, s, prob, q, k, v):
    lib, dev = bsr.library(), q.device
    o = _nan_like(q)
    m = _nan_like(q, torch.float32, q.shape[:3])
    l_ = _nan_like(q, torch.float32, q.shape[:3])
    ws, nbytes = bsr._workspace(s, prob, 0, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    bsr._check(getattr(lib, entry)(s.handle, s.device_plan(dev).data_ptr(), ctypes.byref(prob), q.data_ptr(),
                                   k.data_ptr(), v.data_ptr(), o.data_ptr(), m.data_ptr(), l_.data_ptr(),
                                   bsr._ptr(ws), nbytes, stream))
    return o, m, l_


def _backward(entry, kind, s, prob, q, k, v, o, do, m, l_):
    lib, dev = bsr.library(), q.device
    dq, dk, dv = _nan_like(q), _nan_like(q), _nan_like(q)
    ws, nbytes = bsr._workspace(s, prob, kind, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    bsr._check(getattr(lib, entry)(s.handle, s.device_plan(dev).data_ptr(), ctypes.byref(prob), q.data_ptr(),
                                   k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), m.data_ptr(),
                                   l_.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), bsr._ptr(ws), nbytes,
                                   stream))
    return dq, dk, dv


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("fp32", 128), ("bf16", 64), ("bf16", 128), ("fp16", 128),
                                     ("bf16", 256), ("bf16", 96), ("bf16", 512), ("fp16", 512)])
@pytest.mark.parametrize("nb", [1, 3])
def test_all_empty_mask(dtype, D, nb):
    print(f"all-empty mask: dtype={dtype} D={D} nb={nb}", flush=True)
    bm = np.zeros((nb, nb), dtype=bool)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    assert s.info["nnzb"] == 0
    S = nb * W.BLOCK
    q, k, v, do = W.make_inputs(1, 2, S, D, dtype, seed=7)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    prob = bsr._problem(qd, None)

    # the oracle's plain definition on the same empty structure
    o_r, m_r, l_r = oracle.fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                                  rp, ci)
    assert np.all(o_r == 0) and np.all(np.isneginf(m_r)) and np.all(l_r == 0)
    assert np.all(dq_r == 0) and np.all(dk_r == 0) and np.all(dv_r == 0)

    forwards = ["bsr_attn_fwd", "bsr_attn_fwd_two_pass"]
    backwards = [("bsr_attn_bwd", 1)] + ([("bsr_attn_bwd_ds", 2)] if dtype != "fp32" else [])
    for fe in forwards:
        o, m, l_ = _forward(fe, s, prob, qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.all(o == 0).item(), f"{fe}: O not all zero"
        assert torch.all(torch.isneginf(m)).item(), f"{fe}: row_max not all -inf"
        assert torch.all(l_ == 0).item(), f"{fe}: row_denom not all zero"
        for be, kind in backwards:
            dq, dk, dv = _backward(be, kind, s, prob, qd, kd, vd, o, dod, m, l_)
            torch.cuda.synchronize()
            for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
                assert torch.all(t == 0).item(), f"{fe} -> {be}: {name} not all zero"
