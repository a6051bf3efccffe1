"""The ceiling probes on the GPU: the streaming read must read every
element once (its sums are exact on a buffer of ones), and the MFMA loop
must run every MFMA (its accumulators end at exactly 32 per round)."""
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


@pytest.mark.parametrize("iters,blocks", [(1, 1), (1000, 64), (1 << 19, 2)])
def test_mfma_loop_runs_every_round(iters, blocks):
    out = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    B.moe_probe_mfma_loop(iters, out, blocks)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 32.0 * iters).all()
