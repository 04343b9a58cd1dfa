"""The read-ceiling probe (emb_probe_reads, a measurement aid of bench.py
--ceiling): it reads only inside the buffer it is given and every block's
value is the sum of what lane 0 read (4 columns of `reads` rows of ones)."""
import pytest
import torch

from dlrm_sparse_embedding_amd import emb as E

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("nrows,stride", [(64, 512), (1024, 51200)])
def test_probe_reads_inside_buffer(local, nrows, stride):
    print(f"[gpu] probe nrows={nrows} stride={stride} local={local}", flush=True)
    nbytes = (nrows - 1) * stride + 512
    buf = torch.ones((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    sink = torch.full((E.emb_probe_blocks(),), -1.0, dtype=torch.float32, device="cuda")
    reads = 16
    E.emb_probe_reads(buf, nrows, stride, local, reads, sink)
    torch.cuda.synchronize()
    assert torch.all(sink == 4.0 * reads)
