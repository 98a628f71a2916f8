"""GPU parity of the dS-storing backward (dK/dV stores dS; dQ = dS K is read
from it) against the fp64 oracle at the same tolerances as the recomputing
backward, and its agreement with that backward."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"bf16": 2e-2, "fp16": 2e-3}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def _run(bm, heads, D, dtype, seed=0, split=0):
    rp, ci = W.bsr_from_block_mask(bm)
    S = bm.shape[0] * W.BLOCK
    q, k, v, do = W.make_inputs(1, heads, S, D, dtype, seed)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    grads_ds = bsr.bsr_attn_bwd_ds(s, qd, kd, vd, o, dod, m, l_)
    grads = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
    torch.cuda.synchronize()
    np_ = lambda t: t.float().cpu().double().numpy()
    return rp, ci, (q, k, v, do), [np_(g) for g in grads_ds], [np_(g) for g in grads]


def check(bm, heads, D, dtype, seed=0, split=0):
    rp, ci, (q, k, v, do), ds, ref_gpu = _run(bm, heads, D, dtype, seed, split)
    refs = oracle.bwd(*(t.double().numpy() for t in (q, k, v, do)), rp, ci)
    errs = {}
    for name, g, r, g1 in zip(("dQ", "dK", "dV"), ds, refs, ref_gpu):
        errs[name] = rel(g, r)
        errs[name + " vs bwd"] = rel(g, g1)
    print({k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{n}: {e:.3e}"
    # dV does not depend on dS: the two schedules compute it the same way
    assert np.array_equal(ds[2], ref_gpu[2])
    return ds


@pytest.mark.parametrize("dtype,D", [("bf16", 32), ("bf16", 64), ("bf16", 128), ("bf16", 256), ("fp16", 64),
                                     ("fp16", 128), ("fp16", 256)])
@pytest.mark.parametrize("kind", ["global", "dilated", "random"])
def test_bwd_ds_structures(dtype, D, kind):
    check(W.block_mask(kind, 6, density=0.3, seed=3), 2, D, dtype, seed=1)


@pytest.mark.parametrize("split", [1, 2, 3, 5])
def test_bwd_ds_split_segments(split):
    check(W.block_mask("global", 7), 2, 128, "bf16", seed=2, split=split)


def test_bwd_ds_empty_rows_and_columns():
    bm = np.zeros((4, 4), dtype=bool)
    bm[0, 0] = bm[2, 0] = bm[2, 2] = bm[3, 3] = bm[0, 3] = True  # block row 1 empty; column 1 unreferenced
    dq, dk, dv = check(bm, 2, 64, "bf16", seed=3, split=1)
    sl = slice(W.BLOCK, 2 * W.BLOCK)
    assert np.all(dq[:, :, sl] == 0) and np.all(dk[:, :, sl] == 0) and np.all(dv[:, :, sl] == 0)


@pytest.mark.parametrize("dtype,D", [("bf16", 96), ("fp16", 48)])
def test_bwd_ds_padded_head_dim(dtype, D):
    check(W.block_mask("global", 5), 2, D, dtype, seed=4, split=2)


def test_bwd_ds_deterministic():
    bm = W.block_mask("random", 8, density=0.4, seed=5)
    a = _run(bm, 2, 128, "bf16", seed=6)[3]
    b = _run(bm, 2, 128, "bf16", seed=6)[3]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_ds_rejects_fp32():
    bm = W.block_mask("local", 2)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev).contiguous() for t in W.make_inputs(1, 1, 256, 64, "fp32", 0))
    o, m, l_ = bsr.bsr_attn_fwd(s, q, k, v)
    with pytest.raises(Exception, match="bf16 or fp16"):
        bsr.bsr_attn_bwd_ds(s, q, k, v, o, do, m, l_)


def _sample(S, BH, rng, n_per_head, heads):
    hs = sorted(set([0, BH - 1] + list(rng.integers(0, BH, size=heads))))
    flat = []
    for h in hs:
        picks = [0, 127, S - 1, int(rng.integers(128, 256))] + list(rng.integers(0, S, size=n_per_head))
        flat += [h * S + int(p) for p in picks]
    return np.array(sorted(set(flat)), dtype=np.int64)


@pytest.mark.parametrize("name", ["c3_bf16_global", "c4_bf16_rand10_d256", "c5_bf16_rand50"])
def test_bwd_ds_benchmark_workloads_sampled(name):
    """Full-size workloads in the launch configuration the benchmark times:
    sampled dQ rows and dK/dV keys against the oracle, whole tensors against
    the recomputing backward."""
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[name]
    bm = W.config_mask(name)
    rp, ci, (q, k, v, do), ds, ref_gpu = _run(bm, heads, D, dtype, seed=0)
    inp = [t.double().numpy() for t in (q, k, v, do)]
    rng = np.random.default_rng(7)
    BH = batch * heads
    rows = _sample(S, BH, rng, 4, 3)
    keys = _sample(S, BH, rng, 2, 2)
    flat = lambda x: x.reshape(-1, x.shape[-1])
    dq_r = oracle.bwd_rows(*inp, rp, ci, rows)
    dk_r, dv_r = oracle.bwd_cols(*inp, rp, ci, keys)
    errs = {"dQ": rel(flat(ds[0])[rows], dq_r), "dK": rel(flat(ds[1])[keys], dk_r),
            "dV": rel(flat(ds[2])[keys], dv_r)}
    for n, g, g1 in zip(("dQ", "dK", "dV"), ds, ref_gpu):
        errs[n + " vs bwd"] = rel(g, g1)
    print(name, {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{name}: {n} {e:.3e}"
