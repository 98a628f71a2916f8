"""GPU parity of the block-sparse times dense product (C = A B on the
attention structure's plan) against the fp64 oracle.

Tolerance per output, Frobenius relative error: 1e-5 for fp32 (fp32 matrix
products of exact inputs), 1e-2 for bf16 and 2e-3 for fp16 (the inputs are
exactly representable; products are accumulated in fp32 and C is rounded once
to the operand dtype, unit roundoff 2^-9 and 2^-11)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TOL = {"fp32": 1e-5, "bf16": 1e-2, "fp16": 2e-3}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def run(bm, n_cols, dtype, seed=0, split=0):
    rp, ci = W.bsr_from_block_mask(bm)
    nb = bm.shape[0]
    g = torch.Generator().manual_seed(seed)
    blocks = torch.randn((len(ci), 128, 128), generator=g).to(TDT[dtype]).float()
    b = torch.randn((nb * 128, n_cols), generator=g).to(TDT[dtype]).float()
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    dev = torch.device("cuda:0")
    c = bsr.bsr_spmm(s, blocks.to(dev, TDT[dtype]).contiguous(), b.to(dev, TDT[dtype]).contiguous())
    torch.cuda.synchronize()
    ref = oracle.spmm(blocks.double().numpy(), b.double().numpy(), rp, ci)
    return c.float().cpu().double().numpy(), ref


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("kind,nb,n_cols", [("random", 6, 128), ("global", 5, 256), ("dilated", 8, 384)])
def test_spmm_full(dtype, kind, nb, n_cols):
    c, ref = run(W.block_mask(kind, nb, density=0.35, seed=4), n_cols, dtype, seed=1)
    e = rel(c, ref)
    print(kind, dtype, f"{e:.2e}", flush=True)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("split", [1, 2, 3])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_spmm_split_rows(dtype, split):
    c, ref = run(W.block_mask("global", 7), 256, dtype, seed=2, split=split)
    assert rel(c, ref) <= TOL[dtype]


def test_spmm_wide_tiles():
    """A grid that fills the GPU: many row items times many column tiles."""
    c, ref = run(W.block_mask("random", 40, density=0.05, seed=6), 1664, "bf16", seed=5)
    assert rel(c, ref) <= TOL["bf16"]


def test_spmm_empty_rows_and_no_blocks():
    bm = np.zeros((4, 4), dtype=bool)
    bm[0, 0] = bm[2, 1] = bm[2, 3] = True  # block rows 1 and 3 empty
    c, ref = run(bm, 128, "bf16", seed=3, split=1)
    assert np.all(c[128:256] == 0) and np.all(c[384:] == 0)
    assert rel(c, ref) <= TOL["bf16"]
    s = bsr.bsr_attn_build_structure(np.zeros(3, dtype=np.int32), np.zeros(0, dtype=np.int32))
    b = torch.randn(256, 128, device="cuda:0")
    c0 = bsr.bsr_spmm(s, torch.empty((0, 128, 128), device="cuda:0"), b)
    torch.cuda.synchronize()
    assert torch.all(c0 == 0)


def test_spmm_benchmark_shape_sampled():
    """The pages' SpMM benchmark shape: n = 8192, width 512, 10 % random
    blocks (+ diagonal), bf16, against the oracle's full product."""
    bm = W.block_mask("random", 64, density=0.10, seed=0)
    rp, ci = W.bsr_from_block_mask(bm)
    g = torch.Generator().manual_seed(0)
    blocks = torch.randn((len(ci), 128, 128), generator=g).to(torch.bfloat16)
    b = torch.randn((8192, 512), generator=g).to(torch.bfloat16)
    s = bsr.bsr_attn_build_structure(rp, ci)
    dev = torch.device("cuda:0")
    c = bsr.bsr_spmm(s, blocks.to(dev), b.to(dev)).float().cpu().double().numpy()
    ref = oracle.spmm(blocks.double().numpy(), b.double().numpy(), rp, ci)  # ~8 GFLOP in fp64
    rows = np.unique(np.concatenate([[0, 127, 8191], np.random.default_rng(1).integers(0, 8192, 64)]))
    assert rel(c[rows], ref[rows]) <= TOL["bf16"]
    assert rel(c, ref) <= TOL["bf16"]
