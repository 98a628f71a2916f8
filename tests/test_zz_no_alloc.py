"""GPU: the no-allocation backward (bsr_attn_bwd_noalloc, through the C ABI)
against bsr_attn_bwd with a caller workspace, on two calls in a row, the
second smaller than the first: the library's fixed device workspace keeps
the first call's contents, and the second must not depend on them. Both
entry points run the same kernels, so the gradients must be bit-identical."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(kind, batch, heads, nb, D, dtype, seed, split=0, density=None):
    bm = W.block_mask(kind, nb, density=density, seed=seed)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    q, k, v, do = W.make_inputs(batch, heads, nb * 128, D, dtype, seed)
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev, TDT[dtype]).contiguous() for t in (q, k, v, do))
    o, m, l_ = bsr.bsr_attn_fwd(s, qd, kd, vd)
    return s, (qd, kd, vd, o, dod, m, l_)


def _check(s, args):
    ref = bsr.bsr_attn_bwd(s, *args)
    got = bsr.bsr_attn_bwd_noalloc(s, *args)
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), f"{name} differs from bsr_attn_bwd"


@pytest.mark.parametrize("second", ["bf16_small", "fp32_small_split"])
def test_two_calls_second_smaller(second):
    # first: the 16-head, 8192-token global mask (25 MiB of workspace:
    # delta, lse2 and the partials of the split row 0 and column 0)
    print("[no_alloc] first call: global 1x16x8192x128 bf16", flush=True)
    s1, a1 = _case("global", 1, 16, 64, 128, "bf16", seed=0)
    _check(s1, a1)
    del a1
    print(f"[no_alloc] second call: {second}", flush=True)
    if second == "bf16_small":
        s2, a2 = _case("dilated", 1, 2, 16, 64, "bf16", seed=1)
    else:
        s2, a2 = _case("global", 2, 3, 6, 64, "fp32", seed=2, split=2)
    _check(s2, a2)


def test_head_dim_256_split_columns():
    """head_dim 256 (the two-role kernels) with split rows and columns, after
    a larger call has left its contents in the fixed workspace."""
    print("[no_alloc] first call: random 10 % 1x4x4096x256 bf16", flush=True)
    s1, a1 = _case("random", 1, 4, 32, 256, "bf16", seed=5, density=0.1)
    _check(s1, a1)
    del a1
    print("[no_alloc] second call: global 1x2x1024x256 fp16, split 2", flush=True)
    s2, a2 = _case("global", 1, 2, 8, 256, "fp16", seed=6, split=2)
    _check(s2, a2)


def test_small_launch_on_the_finer_split():
    """One head of four block rows runs on the structure's finer split (every
    row and column merged from one-block segments)."""
    s, a = _case("local", 1, 1, 4, 64, "fp32", seed=3)
    assert s.info["fine_split_threshold"] == 1
    _check(s, a)


def test_too_large_is_rejected_before_launch():
    bm = W.block_mask("global", 64)
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(bm))
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 48, 8192, 128, device=dev, dtype=torch.bfloat16)  # 75 MiB of workspace
    m = torch.zeros(1, 48, 8192, device=dev)
    with pytest.raises(bsr.BsrAttnError, match="WORKSPACE_TOO_SMALL"):
        bsr.bsr_attn_bwd_noalloc(s, q, q, q, q, q, m, m)
