"""The ceiling probes (emb_probe_reads and emb_probe_update, measurement aids
of bench.py --ceiling): the read probe reads only inside the buffer it is
given and every block's value is the sum of what lane 0 read (4 columns of
`reads` rows of ones); the update probe writes only rows of its two row
buffers and leaves its source unchanged."""
import pytest
import torch

from dlrm_sparse_embedding_amd import emb as E

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("nrows,stride,row_bytes", [(64, 512, 512), (1024, 51200, 512), (64, 256, 256),
                                                    (1024, 25600, 256)])
def test_probe_reads_inside_buffer(local, nrows, stride, row_bytes):
    print(f"[gpu] probe nrows={nrows} stride={stride} row={row_bytes} local={local}", flush=True)
    nbytes = (nrows - 1) * stride + row_bytes
    buf = torch.ones((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    sink = torch.full((E.emb_probe_blocks(),), -1.0, dtype=torch.float32, device="cuda")
    reads = 16
    E.emb_probe_reads(buf, nrows, stride, local, reads, sink, row_bytes=row_bytes)
    torch.cuda.synchronize()
    assert torch.all(sink == 4.0 * reads)


def test_probe_update_writes_inside_its_rows():
    print("[gpu] update probe", flush=True)
    nsrc, nrows, items, guard = 300, 200, 5000, 4096
    src = torch.ones(nsrc * 128, dtype=torch.float32, device="cuda")
    a = torch.zeros(nrows * 128 + guard, dtype=torch.float32, device="cuda")
    b = torch.zeros(nrows * 128 + guard, dtype=torch.float32, device="cuda")
    E.emb_probe_update(src, nsrc, a, b, nrows, items)
    torch.cuda.synchronize()
    assert torch.all(src == 1.0)
    assert torch.all(a[nrows * 128:] == 0.0) and torch.all(b[nrows * 128:] == 0.0)
    rows_b = b[: nrows * 128].view(nrows, 128)
    touched = (rows_b != 0.0).any(dim=1)
    assert int(touched.sum()) > nrows // 2
    # every touched state value is a sum of squared gradients of 2 or 3 ones
    assert torch.all(torch.isfinite(rows_b)) and torch.all(rows_b >= 0.0)
    assert torch.all(rows_b[touched] >= 4.0)
    assert torch.all(torch.isfinite(a))
