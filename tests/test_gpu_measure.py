"""The matrix-core ceiling kernel behind comba_mfma_peak_probe computes what
its header says: every wavefront accumulates `iters` times, in four chains,
D = A(16x32) B(32x16) with lane l holding row l % 16 of A and column l % 16 of
B over the same 8 reduction positions, and each thread writes the sum of its
four chains' D rows 4 (l / 16) + 0..3 of column l % 16. The operand values are
multiples of 1/16 and the sums stay far below 2^24 / 128, so every value is
exact in fp32 and the comparison is exact."""
import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def expected_sink(blocks, iters):
    lane = np.arange(64)
    j = np.arange(8)
    a = ((lane[:, None] + j[None, :]) & 7) * 0.125          # lane l's 8 A values
    b = ((lane[:, None] * 3 + j[None, :]) & 7) * 0.0625     # lane l's 8 B values
    # reduction position (g, j) with g = l // 16; A row r = l % 16, B column c = l % 16
    A = np.zeros((16, 32))
    Bm = np.zeros((32, 16))
    for l in range(64):
        g, r = divmod(l, 16)
        A[r, 8 * g:8 * g + 8] = a[l]
        Bm[8 * g:8 * g + 8, r] = b[l]
    D = A @ Bm
    per_lane = np.array([4 * iters * D[4 * (l // 16):4 * (l // 16) + 4, l % 16].sum() for l in range(64)])
    return np.tile(per_lane, blocks * 4)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 64), (300, 17)])
def test_mfma_peak_probe_values(blocks, iters):
    print(f"mfma_peak_probe blocks={blocks} iters={iters}", flush=True)
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flops = comba.mfma_peak_probe(sink, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 4 * 16384
    np.testing.assert_array_equal(sink.cpu().numpy().astype(np.float64), expected_sink(blocks, iters))
