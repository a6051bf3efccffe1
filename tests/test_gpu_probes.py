"""The ceiling probes on the GPU: the streaming read must read every
element once (its sums are exact on a buffer of ones), the row gather must
read every listed row whole (its per-wave sums are exact on small integer
rows), and the MFMA loop and the GEMM K-slice probe must run every MFMA
(their accumulators end at exact multiples of the per-MFMA sum)."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_22_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,blocks", [(4, 1), (1 << 20, 7), ((1 << 22) + 4 * 999, 300)])
def test_stream_read_reads_every_element(n, blocks):
    buf = torch.ones(n, dtype=torch.float32, device="cuda")
    buf[::1024] = 2.0   # marks spread over the buffer
    sums = torch.full((blocks,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_probe_stream_read(buf, n, sums, blocks)
    torch.cuda.synchronize()
    s = sums.cpu().numpy().astype(np.float64)
    assert (s >= 0).all()
    assert s.sum() == n + len(range(0, n, 1024))


@pytest.mark.parametrize("n,blocks", [(4096, 1), (1 << 20, 8), (300 * 4096, 300)])
def test_stream_read_lds_reads_every_element(n, blocks):
    buf = torch.ones(n, dtype=torch.float32, device="cuda")
    buf[::1000] = 3.0
    sums = torch.full((blocks,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_probe_stream_read_lds(buf, n, sums, blocks)
    torch.cuda.synchronize()
    per = n // blocks
    want = [per + 2 * len(range((b * per + 999) // 1000 * 1000, (b + 1) * per, 1000))
            for b in range(blocks)]
    assert np.array_equal(sums.cpu().numpy().astype(np.float64), np.array(want, np.float64))


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("n,blocks", [(8192, 1), (1 << 20, 8), (300 * 8192, 300)])
def test_stream_read_blocks_reads_every_element(n, blocks, nt):
    buf = torch.ones(n, dtype=torch.float32, device="cuda")
    buf[::1000] = 3.0
    sums = torch.full((blocks,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_probe_stream_read_blocks(buf, n, sums, blocks, nt)
    torch.cuda.synchronize()
    per = n // blocks
    want = [per + 2 * len(range((b * per + 999) // 1000 * 1000, (b + 1) * per, 1000))
            for b in range(blocks)]
    assert np.array_equal(sums.cpu().numpy().astype(np.float64), np.array(want, np.float64))


@pytest.mark.parametrize("mode,iters,blocks", [(0, 1, 1), (0, 300, 7), (1, 300, 7), (2, 1, 3),
                                               (2, 300, 256), (3, 1, 3), (3, 300, 256)])
def test_gemm_slice_runs_every_mfma(mode, iters, blocks):
    # every 16-byte LDS chunk starts as bf16 (1, 1, 1, 1, 0, 0, 0, 0): an MFMA
    # over such fragments adds 16 to each accumulator; the copies of modes 2
    # and 3 bring all-ones rows (an MFMA then adds 32) from the second K tile on
    rows = 4096
    src = torch.ones(rows * 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full((blocks,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_probe_gemm_slice(mode, src, rows, iters, out, blocks)
    torch.cuda.synchronize()
    want = 32.0 * iters if mode < 2 else 32.0 + 64.0 * (iters - 1)
    assert (out.cpu().numpy() == want).all()


@pytest.mark.parametrize("iters,blocks", [(1, 1), (1000, 64), (1 << 19, 2)])
def test_mfma_loop_runs_every_round(iters, blocks):
    out = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    B.moe_probe_mfma_loop(iters, out, blocks)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 32.0 * iters).all()


@pytest.mark.parametrize("row_bytes,per,n_waves", [(1024, 1, 5), (2048, 32, 37), (8192, 13, 9)])
def test_row_gather_reads_every_row(row_bytes, per, n_waves):
    n_rows = 300
    rf = row_bytes // 4
    rng = np.random.default_rng(row_bytes + per)
    # row r holds r in every float but one marked element, so a skipped unit
    # or row changes the sum
    table = np.repeat(np.arange(n_rows, dtype=np.float32)[:, None], rf, axis=1)
    table[:, rf // 3] += 1.0
    idx = rng.integers(0, n_rows, size=n_waves * per).astype(np.int32)
    idx[0] = n_rows + 5   # clamped to the last row
    sums = torch.full((n_waves,), -1.0, dtype=torch.float32, device="cuda")
    B.moe_probe_row_gather(torch.from_numpy(table).cuda(), n_rows, row_bytes,
                           torch.from_numpy(idx).cuda(), idx.size, per, sums)
    torch.cuda.synchronize()
    rows = np.clip(idx, 0, n_rows - 1).astype(np.float64).reshape(n_waves, per)
    want = (rows * rf + 1.0).sum(axis=1)
    assert np.array_equal(sums.cpu().numpy().astype(np.float64), want)
