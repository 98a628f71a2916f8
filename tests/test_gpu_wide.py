"""GPU parity of head_dim 512 (the forward in two passes on the fused kernels,
the backward with its gradient blocks materialised and products over the
stored blocks) against the fp64 oracle, and of head dims padded to it."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"bf16": 2e-2, "fp16": 2e-3}
TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def run(bm, batch, heads, D, dtype, seed=0, split=0):
    rp, ci = W.bsr_from_block_mask(bm)
    S = bm.shape[0] * W.BLOCK
    q, k, v, do = W.make_inputs(batch, heads, S, D, dtype, seed)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    grads = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
    torch.cuda.synchronize()
    np_ = lambda t: t.float().cpu().double().numpy()
    out = {"o": np_(o), "m": np_(m), "l": np_(l_), "dq": np_(grads[0]), "dk": np_(grads[1]), "dv": np_(grads[2])}
    return rp, ci, s, (qd, kd, vd, dod, o, m, l_), [t.double().numpy() for t in (q, k, v, do)], out


def check(bm, batch, heads, D, dtype, seed=0, split=0):
    rp, ci, s, dev_t, inp, out = run(bm, batch, heads, D, dtype, seed, split)
    o_r, m_r, l_r = oracle.fwd(inp[0], inp[1], inp[2], rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(*inp, rp, ci)
    fin = np.isfinite(m_r)
    assert np.array_equal(np.isfinite(out["m"]), fin)
    errs = {"O": rel(out["o"], o_r), "row_max": rel(out["m"][fin], m_r[fin]), "row_denom": rel(out["l"], l_r),
            "dQ": rel(out["dq"], dq_r), "dK": rel(out["dk"], dk_r), "dV": rel(out["dv"], dv_r)}
    print({k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{n} rel err {e:.3e} > {TOL[dtype]}"
    return s, dev_t, out


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("kind", ["global", "dilated", "random"])
def test_head_dim_512_structures(dtype, kind):
    check(W.block_mask(kind, 5, density=0.3, seed=3), 1, 2, 512, dtype, seed=1)


@pytest.mark.parametrize("split", [1, 2, 3])
def test_head_dim_512_split_segments(split):
    check(W.block_mask("global", 6), 1, 2, 512, "bf16", seed=2, split=split)


def test_head_dim_512_empty_rows_and_columns():
    bm = np.zeros((4, 4), dtype=bool)
    bm[0, 0] = bm[2, 0] = bm[2, 2] = bm[3, 3] = bm[0, 3] = True  # block row 1 empty; column 1 unreferenced
    _, _, out = check(bm, 1, 2, 512, "bf16", seed=3, split=1)
    sl = slice(W.BLOCK, 2 * W.BLOCK)
    assert np.all(out["o"][:, :, sl] == 0) and np.all(np.isneginf(out["m"][:, :, sl]))
    assert np.all(out["dq"][:, :, sl] == 0) and np.all(out["dk"][:, :, sl] == 0) and np.all(out["dv"][:, :, sl] == 0)


def test_head_dim_512_batch_and_other_entry_points():
    """Several (batch, head) pairs; the two-pass forward and the dS-storing
    backward at this width run the same path and agree exactly."""
    s, (q, k, v, do, o, m, l_), _, = check(W.block_mask("random", 4, density=0.4, seed=4), 2, 3, 512, "bf16", seed=5)[:3]
    o2, m2, l2 = bsr.bsr_attn_fwd_two_pass(s, q, k, v)
    g1 = bsr.bsr_attn_bwd(s, q, k, v, o, do, m, l_)
    g2 = bsr.bsr_attn_bwd_ds(s, q, k, v, o, do, m, l_)
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(m2, m) and torch.equal(l2, l_)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D", [("bf16", 384), ("fp16", 272)])
def test_head_dims_padded_to_512(dtype, D):
    check(W.block_mask("global", 4), 1, 2, D, dtype, seed=6, split=2)


def test_head_dim_512_deterministic():
    bm = W.block_mask("random", 5, density=0.4, seed=7)
    a = run(bm, 1, 2, 512, "bf16", seed=8)[-1]
    b = run(bm, 1, 2, 512, "bf16", seed=8)[-1]
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_head_dim_512_longer_sequence_sampled():
    """seq 4096 (32 block rows), 4 heads, random 10 % + diagonal: sampled rows
    and keys against the oracle."""
    bm = W.block_mask("random", 32, density=0.10, seed=0)
    rp, ci, s, _, inp, out = run(bm, 1, 4, 512, "bf16", seed=0)
    S = 32 * W.BLOCK
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set([0, 127, S - 1, S + 5, 3 * S + 200] + list(rng.integers(0, 4 * S, size=6)))))
    keys = np.array(sorted(set([1, S - 2, 2 * S + 7] + list(rng.integers(0, 4 * S, size=4)))))
    flat = lambda x: x.reshape(-1, x.shape[-1]) if x.ndim == 4 else x.reshape(-1)
    o_r, m_r, l_r = oracle.fwd_rows(inp[0], inp[1], inp[2], rp, ci, rows)
    dq_r = oracle.bwd_rows(*inp, rp, ci, rows)
    dk_r, dv_r = oracle.bwd_cols(*inp, rp, ci, keys)
    errs = {"O": rel(flat(out["o"])[rows], o_r), "row_max": rel(flat(out["m"])[rows], m_r),
            "row_denom": rel(flat(out["l"])[rows], l_r), "dQ": rel(flat(out["dq"])[rows], dq_r),
            "dK": rel(flat(out["dk"])[keys], dk_r), "dV": rel(flat(out["dv"])[keys], dv_r)}
    print({k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= TOL["bf16"], f"{n} {e:.3e}"


@pytest.mark.parametrize("split", [0, 2])
def test_head_dim_512_growing_row_max(split):
    """Key blocks with growing norms push each row's maximum up block after
    block (head 0) or put it first (head 1): the statistics pass rescales its
    running sum, the output pass uses the final statistics, and the backward
    forms P from them; all must match the oracle."""
    nb, D = 5, 512
    bm = W.block_mask("full", nb)
    rp, ci = W.bsr_from_block_mask(bm)
    S = nb * W.BLOCK
    q, k, v, do = W.make_inputs(1, 2, S, D, "bf16", seed=12)
    growth = torch.ones(S)
    for j in range(nb):
        growth[j * W.BLOCK:(j + 1) * W.BLOCK] = 1.0 + 1.5 * j
    k = (k * growth[None, None, :, None]).to(torch.bfloat16).float()
    k[:, 1] = k[:, 1].flip(2)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, torch.bfloat16).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    dq, dk, dv = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
    torch.cuda.synchronize()
    inp = [t.double().numpy() for t in (q, k, v, do)]
    o_r, m_r, l_r = oracle.fwd(*inp[:3], rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(*inp, rp, ci)
    for name, x, ref in (("O", o, o_r), ("row_max", m, m_r), ("row_denom", l_, l_r),
                         ("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
        e = rel(x.float().cpu().double().numpy(), ref)
        assert e <= TOL["bf16"], f"{name} rel err {e:.3e}"
    # head 0: the row max grows well past the first key block's
    first = (inp[0][0, 0] @ inp[1][0, 0, :W.BLOCK].T / np.sqrt(D)).max(axis=1)
    assert np.median(m_r[0, 0] - first) * np.log2(np.e) > 16.0
