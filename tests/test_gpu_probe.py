"""GPU: the MFMA-loop probe the benchmark uses for its measured peak runs,
reports the matrix work it launched, and leaves its sink alone."""
import pytest
import torch

pytestmark = pytest.mark.gpu
bsr = pytest.importorskip("block_sparse_attention_bsr_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,k", [(torch.bfloat16, 16), (torch.float16, 16), (torch.float32, 2)])
def test_mfma_probe(dtype, k):
    sink = torch.zeros(1, device="cuda:0")
    iters = 64
    flops = bsr.mfma_probe(dtype, iters, sink)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    # two 4-wave workgroups per CU, 4 chains of `iters` 32x32xk products per wave
    assert flops == 2 * cus * 4 * 4 * iters * 2 * 32 * 32 * k
    assert sink.item() == 0.0


def test_mfma_probe_rejects_bad_arguments():
    sink = torch.zeros(1, device="cuda:0")
    with pytest.raises(Exception):
        bsr.mfma_probe(torch.bfloat16, 0, sink)
    with pytest.raises(TypeError):
        bsr.mfma_probe(torch.int32, 8, sink)
