"""bench.py's measurement probes move the right bytes: a plain gather (plain and
non-temporal loads) and scatter of random rows (measure/libprobes.so) against torch
indexing, in HBM and between pinned host memory and HBM, with a ragged last round, and
a contiguous copy (both loads) that stops at its end."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("row_bytes,n,pool,blocks,host", [
    (656, 1000, 5000, 3, False),
    (1968, 777, 2000, 96, True),
    (16, 70001, 90000, 1024, True),
])
def test_move_rows_gather_and_scatter(row_bytes, n, pool, blocks, host):
    import torch
    from measure import probes
    torch.cuda.set_device(0)
    rng = np.random.default_rng(n)
    idx_np = rng.permutation(pool)[:n].astype(np.int32)
    idx = torch.from_numpy(idx_np).cuda()
    src = torch.randint(0, 256, (pool, row_bytes), dtype=torch.uint8)
    src = src.pin_memory() if host else src.cuda()
    out = torch.zeros((n, row_bytes), dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    for mode in (0, 2):                       # plain and non-temporal loads
        out.zero_()
        probes.move_rows(mode, src, idx, out, n, row_bytes, blocks, s)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), src.cpu()[torch.from_numpy(idx_np).long()]), mode
    rows = torch.randint(0, 256, (n, row_bytes), dtype=torch.uint8, device="cuda")
    dst = torch.zeros((pool, row_bytes), dtype=torch.uint8)
    dst = dst.pin_memory() if host else dst.cuda()
    probes.move_rows(1, rows, idx, dst, n, row_bytes, blocks, s)
    torch.cuda.synchronize()
    want = torch.zeros((pool, row_bytes), dtype=torch.uint8)
    want[torch.from_numpy(idx_np).long()] = rows.cpu()
    assert torch.equal(dst.cpu(), want)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (656 * 777, 3), (16 * 1_000_003, 1024)])
def test_copy_probe(nbytes, blocks):
    import torch
    from measure import probes
    torch.cuda.set_device(0)
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    for nt in (False, True):                  # plain and non-temporal loads
        dst.zero_()
        probes.copy_bytes(src, dst, nbytes, blocks, torch.cuda.current_stream(), nt=nt)
        torch.cuda.synchronize()
        assert torch.equal(dst[:nbytes], src[:nbytes]), nt
        assert not dst[nbytes:].any(), "copied past its end"
