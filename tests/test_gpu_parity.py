"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small structures are compared in full, element by element. Most full-size
benchmark workloads are compared whole in test_gpu_fullsize.py; the random
masks at 50 % density (about a minute of oracle time per dtype) run here in
the launch configuration the benchmark times and are compared on sampled query
rows (O, row_max, row_denom, dQ) and sampled keys (dK, dV) that the oracle
computes one by one, plus properties that hold at any size.

Tolerance: per output tensor, the Frobenius relative error
||x - ref|| / ||ref|| in fp64, at most 1e-4 for fp32 operands and 2e-2 for
bf16 operands, against the oracle evaluated on the same (dtype-rounded) inputs.
fp16 operands (a dtype the pages name, with no stated tolerance): 2e-3, about
four times fp16's unit roundoff 2^-11, since P, dS and the outputs are each
rounded once to fp16 and every sum is accumulated in fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"fp32": 1e-4, "bf16": 2e-2, "fp16": 2e-3}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
B = W.BLOCK


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsr.library()


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def run(bm, batch, heads, D, dtype, seed=0, split=0, scale=None):
    rp, ci = W.bsr_from_block_mask(bm)
    S = bm.shape[0] * B
    q, k, v, do = W.make_inputs(batch, heads, S, D, dtype, seed)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd, scale=scale)
    dq, dk, dv = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_, scale=scale)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().double().numpy() for n, t in
           (("o", o), ("m", m), ("l", l_), ("dq", dq), ("dk", dk), ("dv", dv))}
    inp = {n: t.double().numpy() for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
    return rp, ci, s, inp, out


def check_full(bm, batch, heads, D, dtype, seed=0, split=0, scale=None):
    rp, ci, s, inp, out = run(bm, batch, heads, D, dtype, seed, split, scale)
    o_r, m_r, l_r = oracle.fwd(inp["q"], inp["k"], inp["v"], rp, ci, scale=scale)
    dq_r, dk_r, dv_r = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["do"], rp, ci, scale=scale)
    tol = TOL[dtype]
    finite = np.isfinite(m_r)
    assert np.array_equal(np.isfinite(out["m"]), finite), "empty-row statistics differ"
    errs = {
        "O": rel(out["o"], o_r), "row_max": rel(out["m"][finite], m_r[finite]), "row_denom": rel(out["l"], l_r),
        "dQ": rel(out["dq"], dq_r), "dK": rel(out["dk"], dk_r), "dV": rel(out["dv"], dv_r),
    }
    print({k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for name, e in errs.items():
        assert e <= tol, f"{name} rel err {e:.3e} > {tol}"
    return out, (o_r, m_r, l_r, dq_r, dk_r, dv_r)


# ---------------------------------------------------------------------------
# Full element-by-element comparisons at small sizes
# ---------------------------------------------------------------------------
def test_config1_fp32_local_full():
    """fp32, 1 x 1 x 512 x 64, local window: the whole output."""
    check_full(W.block_mask("local", 4), 1, 1, 64, "fp32")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("fp32", 64), ("fp32", 128),
                                     ("fp16", 64), ("fp16", 128), ("fp16", 256),
                                     ("bf16", 32), ("fp32", 32), ("fp16", 32)])
@pytest.mark.parametrize("kind", ["global", "dilated", "random"])
def test_structures_full(dtype, D, kind):
    nb = 6
    bm = W.block_mask(kind, nb, density=0.3, seed=3)
    check_full(bm, 1, 2, D, dtype, seed=1)


@pytest.mark.parametrize("dtype,D", [("bf16", 16), ("bf16", 48), ("bf16", 80), ("bf16", 96), ("bf16", 112),
                                     ("bf16", 192), ("fp32", 16), ("fp32", 48), ("fp32", 96), ("fp32", 112),
                                     ("fp16", 48), ("fp16", 160)])
def test_padded_head_dims_full(dtype, D):
    """Head dims without an instance of their own (any multiple of 16) run on
    zero-padded copies at the next instantiated width; forward and backward
    must match the oracle at the real width, split segments included."""
    check_full(W.block_mask("global", 5), 1, 2, D, dtype, seed=12, split=2)


@pytest.mark.parametrize("split", [1, 2, 3, 5])
@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
def test_split_segments_ragged(dtype, split):
    """Long rows/columns split into uneven segments whose partials are merged."""
    bm = W.block_mask("global", 7)
    check_full(bm, 1, 2, 64 if dtype == "fp32" else 128, dtype, seed=2, split=split)


@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
def test_empty_rows_and_columns(dtype):
    bm = np.zeros((4, 4), dtype=bool)
    bm[0, 0] = bm[2, 0] = bm[2, 2] = bm[3, 3] = bm[0, 3] = True  # block row 1 empty; column 1 unreferenced
    out, _ = check_full(bm, 1, 2, 64, dtype, seed=3, split=1)
    sl = slice(B, 2 * B)
    assert np.all(out["o"][:, :, sl] == 0) and np.all(np.isneginf(out["m"][:, :, sl]))
    assert np.all(out["l"][:, :, sl] == 0) and np.all(out["dq"][:, :, sl] == 0)
    assert np.all(out["dk"][:, :, sl] == 0) and np.all(out["dv"][:, :, sl] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("split", [1, 3])
def test_head_dim_256_split_and_empty(dtype, split):
    """head_dim 256 has a forward of its own (roles split over two waves per
    SIMD): ragged splits (partials merged) and an empty block row through it
    and the backward."""
    bm = np.zeros((6, 6), dtype=bool)
    bm[0, :] = True
    bm[2, 0] = bm[2, 2] = bm[3, 3] = bm[4, 1] = bm[4, 4] = bm[5, 5] = bm[5, 0] = True  # block row 1 empty
    out, _ = check_full(bm, 1, 2, 256, dtype, seed=13, split=split)
    sl = slice(B, 2 * B)
    assert np.all(out["o"][:, :, sl] == 0) and np.all(np.isneginf(out["m"][:, :, sl]))
    assert np.all(out["l"][:, :, sl] == 0) and np.all(out["dq"][:, :, sl] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("split", [0, 3])
def test_head_dim_256_dkdv_empty_and_long_columns(dtype, split):
    """head_dim 256 dK/dV (roles split over two waves per SIMD, 32-row stages
    in a four-buffer ring): a key-block column no row references (dK = dV =
    0), a full column (seven blocks: 28 stages, split raggedly at threshold
    3 into 3 + 2 + 2 blocks) and one-block columns (four stages, fewer than
    the ring holds)."""
    nb = 7
    bm = np.zeros((nb, nb), dtype=bool)
    bm[:, 0] = True                      # column 0: every block row
    bm[1, 1] = bm[2, 2] = bm[3, 2] = bm[4, 4] = bm[5, 5] = bm[6, 5] = True  # column 3 and 6: empty
    out, _ = check_full(bm, 1, 2, 256, dtype, seed=17, split=split)
    for c in (3, 6):
        sl = slice(c * B, (c + 1) * B)
        assert np.all(out["dk"][:, :, sl] == 0) and np.all(out["dv"][:, :, sl] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_full_and_diagonal_masks(dtype):
    check_full(W.block_mask("full", 4), 1, 1, 64, dtype, seed=4)
    check_full(W.block_mask("diagonal", 5), 1, 1, 64, dtype, seed=5)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("kind", ["local", "pages_dilated"])
def test_pages_test_shape_head_dim_32(dtype, kind):
    """The pages' simulator and gradcheck shape: seq 256 (2 x 2 blocks),
    head_dim 32, local-window and (the pages' own) dilated masks."""
    if kind == "local":
        bm = W.block_mask("local", 2)
    else:
        bm = np.array([[(j - i) % 4 == 0 for j in range(2)] for i in range(2)])  # stride 4, no band
    check_full(bm, 1, 1, 32, dtype, seed=11)


def test_single_block():
    check_full(np.ones((1, 1), dtype=bool), 1, 1, 128, "bf16", seed=6)


def test_batch_heads_and_custom_scale():
    check_full(W.block_mask("dilated", 6), 2, 3, 128, "bf16", seed=7, scale=0.05)
    check_full(W.block_mask("local", 5), 3, 2, 64, "fp32", seed=8, scale=0.3)


@pytest.mark.parametrize("dtype,D,batch", [("bf16", 64, 4), ("bf16", 128, 2), ("fp16", 128, 2)])
def test_many_heads_one_queue_per_head(dtype, D, batch):
    """More (batch, head) pairs than half the dK/dV pass's workgroup slots
    (256 CUs; two workgroups per CU at head_dim 64): that pass then runs one
    work queue per head, and the others launch several rounds of workgroups."""
    check_full(W.block_mask("global", 3), batch, 80, D, dtype, seed=13, split=2)


def test_sharp_softmax():
    """Large scores: the online max must keep every exponent finite."""
    check_full(W.block_mask("global", 5), 1, 2, 64, "fp32", seed=9, scale=4.0)
    check_full(W.block_mask("global", 5), 1, 2, 128, "bf16", seed=9, scale=2.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("split", [0, 2])
def test_growing_row_max(dtype, split):
    """Key blocks with growing norms push each row's max up block after block
    (by far more than the forward's rescale threshold); rows whose largest
    score comes first never rescale. Both must match the oracle."""
    nb, D = 6, 64
    bm = W.block_mask("full", nb)
    rp, ci = W.bsr_from_block_mask(bm)
    S = nb * B
    q, k, v, do = W.make_inputs(1, 2, S, D, dtype, seed=11)
    growth = torch.ones(S)
    for j in range(nb):
        growth[j * B:(j + 1) * B] = 1.0 + 1.5 * j
    k = (k * growth[None, None, :, None]).to(TDT[dtype]).float()
    k[:, 1] = k[:, 1].flip(2)  # head 1: largest keys first
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    dq, dk, dv = bsr.bsr_attn_bwd(s, qd, kd, vd, o, dod, m, l_)
    torch.cuda.synchronize()
    inp = [t.double().numpy() for t in (q, k, v, do)]
    o_r, m_r, l_r = oracle.fwd(*inp[:3], rp, ci)
    dq_r, dk_r, dv_r = oracle.bwd(*inp, rp, ci)
    tol = TOL[dtype]
    for name, x, ref in (("O", o, o_r), ("row_max", m, m_r), ("row_denom", l_, l_r),
                         ("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r)):
        e = rel(x.float().cpu().double().numpy(), ref)
        assert e <= tol, f"{name} rel err {e:.3e} > {tol}"
    # head 0: the row max must grow well past 2^8 over the first key block's max
    first = (inp[0][0, 0] @ inp[1][0, 0, :B].T / np.sqrt(D)).max(axis=1)
    assert np.median(m_r[0, 0] - first) * np.log2(np.e) > 16.0


@pytest.mark.parametrize("dtype,D,heads", [("bf16", 64, 2), ("fp16", 128, 1)])
@pytest.mark.timeout(200)
def test_long_sequence(dtype, D, heads):
    """A long sequence: 4096 block rows (seq 524288), local window plus a
    global first column, so that row/column offsets, plan indices and the
    split of column 0 (4096 blocks) run at large values. Sampled rows and keys
    against the oracle; the whole-output identities hold everywhere."""
    nb = 4096
    bm = np.zeros((nb, nb), dtype=bool)
    i = np.arange(nb)
    for d in (-1, 0, 1):
        j = i + d
        ok = (j >= 0) & (j < nb)
        bm[i[ok], j[ok]] = True
    bm[:, 0] = True
    rp, ci, s, inp, out = run(bm, 1, heads, D, dtype, seed=9)
    tol = TOL[dtype]
    S = nb * B
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 127, 128, S - 1], rng.integers(0, heads * S, size=24)]))
    # key 0 (block column 0, stored by every row: the oracle walks all 524288
    # query rows for it) and keys of other columns (three block rows each)
    other = rng.integers(B, S, size=12)
    keys = np.unique(np.concatenate([[0, S - 1], other, (heads - 1) * S + other[:4]]))
    flat = lambda x: x.reshape(-1, x.shape[-1]) if x.ndim == 4 else x.reshape(-1)
    o_r, m_r, l_r = oracle.fwd_rows(inp["q"], inp["k"], inp["v"], rp, ci, rows)
    dq_r = oracle.bwd_rows(inp["q"], inp["k"], inp["v"], inp["do"], rp, ci, rows)
    dk_r, dv_r = oracle.bwd_cols(inp["q"], inp["k"], inp["v"], inp["do"], rp, ci, keys)
    errs = {"O": rel(flat(out["o"])[rows], o_r), "row_max": rel(flat(out["m"])[rows], m_r),
            "row_denom": rel(flat(out["l"])[rows], l_r), "dQ": rel(flat(out["dq"])[rows], dq_r),
            "dK": rel(flat(out["dk"])[keys], dk_r), "dV": rel(flat(out["dv"])[keys], dv_r),
            "sum_dV=sum_dO": rel(out["dv"].sum(axis=2), inp["do"].sum(axis=2))}
    print(errs, flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{n} rel err {e:.3e} > {tol}"


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_deterministic(dtype, D):
    bm = W.block_mask("global", 8)
    a = run(bm, 1, 2, D, dtype, seed=10, split=3)[4]
    b = run(bm, 1, 2, D, dtype, seed=10, split=3)[4]
    for n in a:
        assert np.array_equal(a[n], b[n], equal_nan=True), n


def test_config2_dilated_two_heads_full():
    """Config 2's shape per head (bf16, seq 2048, head_dim 128, dilated), 2 of its 8 heads in full."""
    check_full(W.block_mask("dilated", 16), 1, 2, 128, "bf16", seed=0)


# ---------------------------------------------------------------------------
# Full-size configurations: sampled outputs and whole-tensor properties
# ---------------------------------------------------------------------------
def _sample(S, BH, nb, rng, n_per_head=6, heads=4):
    hs = sorted(set([0, BH - 1] + list(rng.integers(0, BH, size=heads))))
    flat = []
    for h in hs:
        picks = [0, 127, S - 1, int(rng.integers(128, 256)), int(rng.integers(0, S))]
        picks += list(rng.integers(0, S, size=max(0, n_per_head - len(picks))))
        flat += [h * S + int(p) for p in picks]
    return np.array(sorted(set(flat)), dtype=np.int64)


CONFIGS = ["c5_fp32_rand50", "c5_bf16_rand50"]


@pytest.mark.parametrize("name", CONFIGS)
def test_benchmark_config_sampled(name):
    dtype, batch, heads, S, D, kind, dens = W.CONFIGS[name]
    bm = W.config_mask(name)
    rp, ci, s, inp, out = run(bm, batch, heads, D, dtype, seed=0)
    tol = TOL[dtype]
    rng = np.random.default_rng(123)
    BH = batch * heads
    rows = _sample(S, BH, bm.shape[0], rng)
    flat = lambda x: x.reshape(-1, x.shape[-1]) if x.ndim == 4 else x.reshape(-1)
    o_r, m_r, l_r = oracle.fwd_rows(inp["q"], inp["k"], inp["v"], rp, ci, rows)
    dq_r = oracle.bwd_rows(inp["q"], inp["k"], inp["v"], inp["do"], rp, ci, rows)
    keys = _sample(S, BH, bm.shape[0], rng, n_per_head=3, heads=2)
    dk_r, dv_r = oracle.bwd_cols(inp["q"], inp["k"], inp["v"], inp["do"], rp, ci, keys)
    errs = {
        "O": rel(flat(out["o"])[rows], o_r), "row_max": rel(flat(out["m"])[rows], m_r),
        "row_denom": rel(flat(out["l"])[rows], l_r), "dQ": rel(flat(out["dq"])[rows], dq_r),
        "dK": rel(flat(out["dk"])[keys], dk_r), "dV": rel(flat(out["dv"])[keys], dv_r),
    }
    # properties over the whole output (every row attends to its diagonal block here)
    dv_sum = out["dv"].sum(axis=2)
    do_sum = inp["do"].sum(axis=2)
    errs["sum_dV=sum_dO"] = rel(dv_sum, do_sum)
    errs["sum_dK=0"] = float(np.linalg.norm(out["dk"].sum(axis=2)) / np.linalg.norm(out["dk"]))
    print(name, {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
    for n, e in errs.items():
        assert e <= tol, f"{name}: {n} rel err {e:.3e} > {tol}"
    assert np.all(np.isfinite(out["o"])) and np.all(np.isfinite(out["dq"]))


def test_concurrent_streams_and_threads():
    """Calls that overlap on two streams, from two host threads, sharing one
    structure (its device plan, read only) while each has its own workspace:
    every result equals the same call made alone. The structure and its
    plan are documented as shareable between threads and streams."""
    import threading

    bm = W.block_mask("global", 8)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=3)
    dev = torch.device("cuda:0")
    jobs = []
    for seed, dtype, D in ((21, "bf16", 128), (22, "fp32", 64)):
        q, k, v, do = W.make_inputs(1, 3, 8 * B, D, dtype, seed)
        jobs.append(tuple(t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do)))

    def step(j):
        q, k, v, do = j
        o, m, l_ = bsr.bsr_attn_fwd(s, q, k, v)
        return (o, m, l_) + bsr.bsr_attn_bwd(s, q, k, v, o, do, m, l_)

    alone = [step(j) for j in jobs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in jobs]  # default priority
    results = [None] * len(jobs)

    def worker(i):
        with torch.cuda.stream(streams[i]):
            for _ in range(3):
                results[i] = step(jobs[i])

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for a, r in zip(alone, results):
        for x, y in zip(a, r):
            assert torch.equal(x, y)
