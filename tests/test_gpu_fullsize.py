"""GPU parity at full size: every output row of the benchmark workloads against
the fp64 oracle.

Each workload runs through the C ABI in the launch configuration the
benchmark times (automatic split threshold, the same seeded inputs), and the
whole O, row_max, row_denom, dQ, dK and dV are compared with the oracle's
forward and backward over the same (dtype-rounded) inputs, as the pages'
attention benchmark compares its whole outputs with a dense fp64 reference
(page "trnsparse 0.7.0 -> 0.9.0", benchmarks/bench_native_trn2.py, attention
section, rel_err of the forward output and of the gradients).

Two gates per tensor, both at the tolerance of the operand dtype (rel 1e-4
fp32, 2e-2 bf16; fp16 2e-3):
  * the pages' relative error of the whole tensor;
  * the worst single row (tests/parity_metrics.py, row_err), so that one
    wrong row among 131072 cannot hide in the whole-tensor figure.
The random masks at 50 % density (oracle time about a minute per dtype) stay
sampled in test_gpu_parity.py. head_dim 512 (its own forward and backward
kernels) is checked whole at the 10 % mask.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_metrics import rel, row_err

pytestmark = pytest.mark.gpu

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 2e-3}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}

FULL = ["c1_fp32_local", "c2_bf16_dilated", "c3_bf16_global", "c4_bf16_rand10_d256"] + [
    f"c5_{dt}_rand{d:02d}" for d in (1, 5, 10, 25) for dt in ("bf16", "fp32")] + ["x_fp16_rand10",
                                                                                  "x_bf16_rand10_d512"]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsr.library()


@pytest.mark.parametrize("name", FULL)
@pytest.mark.timeout(300)
def test_benchmark_config_whole_output(name):
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[name]
    print(f"[fullsize] {name}: {dtype} {batch}x{heads}x{S}x{D} {kind}", flush=True)
    bm = W.config_mask(name)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = W.make_inputs(batch, heads, S, D, dtype, seed=0)
    s = bsr.bsr_attn_build_structure(rp, ci)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    dq, dk, dv = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
    torch.cuda.synchronize()
    gpu = {n: t.float().cpu().double().numpy() for n, t in
           (("O", o), ("row_max", m), ("row_denom", l_), ("dQ", dq), ("dK", dk), ("dV", dv))}
    del qd, kd, vd, dod, o, m, l_, dq, dk, dv
    inp = [t.double().numpy() for t in (q, k, v, do)]
    del q, k, v, do
    o_r, m_r, l_r = oracle.fwd(*inp[:3], rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(*inp, rp, ci)
    ref = {"O": o_r, "row_max": m_r, "row_denom": l_r, "dQ": dq_r, "dK": dk_r, "dV": dv_r}
    # every block row and column of these masks stores its diagonal block
    assert np.all(np.isfinite(m_r)) and np.all(np.isfinite(gpu["row_max"]))
    tol = TOL[dtype]
    errs = {}
    for n in ref:
        errs[n] = (rel(gpu[n], ref[n]), row_err(gpu[n], ref[n]))
    print(name, {n: f"rel {a:.2e} row {b:.2e}" for n, (a, b) in errs.items()}, flush=True)
    for n, (a, b) in errs.items():
        assert a <= tol, f"{name}: {n} rel err {a:.3e} > {tol}"
        assert b <= tol, f"{name}: {n} worst-row err {b:.3e} > {tol}"
