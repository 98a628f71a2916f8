"""GPU parity of the two-pass forward (statistics pass, then output pass)
against the fp64 oracle, at the same tolerances as the one-pass forward, and
its agreement with the one-pass forward."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 2e-3}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def check(bm, heads, D, dtype, seed=0, split=0):
    rp, ci = W.bsr_from_block_mask(bm)
    S = bm.shape[0] * W.BLOCK
    q, k, v, _ = W.make_inputs(1, heads, S, D, dtype, seed)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v))
    o, m, l_ = bsr.bsr_attn_fwd_two_pass(s, qd, kd, vd)
    o1, m1, l1 = bsr.bsr_attn_fwd(s, qd, kd, vd)
    torch.cuda.synchronize()
    o_r, m_r, l_r = oracle.fwd(*(t.double().numpy() for t in (q, k, v)), rp, ci)
    fin = np.isfinite(m_r)
    om, mm, lm = (t.float().cpu().double().numpy() for t in (o, m, l_))
    assert np.array_equal(np.isfinite(mm), fin)
    errs = {"O": rel(om, o_r), "row_max": rel(mm[fin], m_r[fin]), "row_denom": rel(lm, l_r)}
    print(errs, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{n}: {e:.3e}"
    # the statistics pass tracks the same maximum as the one-pass forward
    assert torch.equal(m, m1)
    assert rel(om, o1.float().cpu().double().numpy()) <= TOL[dtype]
    return om, mm, lm


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("fp32", 32), ("bf16", 128), ("bf16", 256), ("bf16", 32),
                                     ("fp16", 64)])
@pytest.mark.parametrize("kind", ["global", "random"])
def test_two_pass_structures(dtype, D, kind):
    check(W.block_mask(kind, 6, density=0.3, seed=3), 2, D, dtype, seed=1)


@pytest.mark.parametrize("dtype,D", [("bf16", 96), ("fp32", 48)])
def test_two_pass_padded_head_dim(dtype, D):
    check(W.block_mask("global", 5), 2, D, dtype, seed=4, split=2)


@pytest.mark.parametrize("split", [1, 3])
def test_two_pass_split_rows(split):
    check(W.block_mask("global", 7), 2, 128, "bf16", seed=2, split=split)


def test_two_pass_empty_rows():
    bm = np.zeros((4, 4), dtype=bool)
    bm[0, 0] = bm[2, 0] = bm[2, 2] = bm[3, 3] = bm[0, 3] = True
    om, mm, lm = check(bm, 2, 64, "fp32", seed=3, split=1)
    sl = slice(W.BLOCK, 2 * W.BLOCK)
    assert np.all(om[:, :, sl] == 0) and np.all(np.isneginf(mm[:, :, sl])) and np.all(lm[:, :, sl] == 0)


def test_two_pass_benchmark_workload_sampled():
    """The 16-head seq-8192 global-mask workload, in the launch configuration
    the benchmark times: sampled rows against the oracle."""
    name = "c3_bf16_global"
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[name]
    bm = W.config_mask(name)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, _ = W.make_inputs(batch, heads, S, D, dtype, seed=0)
    s = bsr.bsr_attn_build_structure(rp, ci)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v))
    o, m, l_ = bsr.bsr_attn_fwd_two_pass(s, qd, kd, vd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 127, S - 1], rng.integers(0, batch * heads * S, size=40)]))
    o_r, m_r, l_r = oracle.fwd_rows(*(t.double().numpy() for t in (q, k, v)), rp, ci, rows)
    of = o.float().cpu().double().numpy().reshape(-1, D)[rows]
    assert rel(of, o_r) <= TOL[dtype]
    assert rel(m.cpu().double().numpy().reshape(-1)[rows], m_r) <= TOL[dtype]
    assert rel(l_.cpu().double().numpy().reshape(-1)[rows], l_r) <= TOL[dtype]
