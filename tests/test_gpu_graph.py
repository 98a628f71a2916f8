"""GPU: the entry points under HIP graph capture.

The launch path allocates nothing and sets no memory itself (the workspace
comes from the caller, here torch's caching allocator, which serves captures
from the graph's own pool), so a forward + backward can be captured once and
replayed. Every replay, with unrelated eager work and synchronisations in
between, must give exactly the eager results; the allocation-free backward
is captured the same way (its fixed device array is what it is for).
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsr.library()


@pytest.mark.parametrize("entry", ["bsr_attn_bwd", "bsr_attn_bwd_noalloc"])
def test_graph_replays_match_eager(entry):
    bm = W.block_mask("global", 8)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=3)  # split rows and columns: merges and sums
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev, torch.bfloat16).contiguous() for t in W.make_inputs(1, 2, 8 * 128, 128, "bf16", seed=31))
    bwd = getattr(bsr, entry)

    def step():
        o, m, l_ = bsr.bsr_attn_fwd(s, q, k, v)
        return (o, m, l_) + bwd(s, q, k, v, o, do, m, l_)

    ref = step()  # eager; also uploads the structure's device plan before capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for rep in range(3):
        junk = torch.randn(1 << 20, device=dev)
        (junk * 2).max().item()  # unrelated eager work and a synchronisation
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("O", "row_max", "row_denom", "dQ", "dK", "dV"), out, ref):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from the eager result"
