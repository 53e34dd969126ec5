"""GPU checks of the measured-peak probes (rpa_probe_read, rpa_probe_mfma).

The probes report what the device sustains, so they must really read every
byte and really run the matrix instructions: each one's output is compared
with a closed form computed on the CPU.
"""
import numpy as np
import pytest
import torch

from gpu_common import gpu_available

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import ragged_paged_attention_forward_amd as R  # noqa: E402


def expected_read_fold(data: np.ndarray, workgroups: int, threads: int = 256) -> np.ndarray:
    """Thread t of workgroup b folds (XOR) the four words of every 16-byte
    chunk b*per_wg + t + threads*i of its slice [b*per_wg, min((b+1)*per_wg, n))."""
    words = data.view(np.uint32).reshape(-1, 4)
    fold = words[:, 0] ^ words[:, 1] ^ words[:, 2] ^ words[:, 3]
    n = fold.shape[0]
    per_wg = -(-n // workgroups)
    cols = -(-per_wg // threads) * threads
    grid = np.zeros((workgroups, cols), dtype=np.uint32)
    for b in range(workgroups):
        lo, hi = b * per_wg, min((b + 1) * per_wg, n)
        if hi > lo:
            grid[b, : hi - lo] = fold[lo:hi]
    return np.bitwise_xor.reduce(grid.reshape(workgroups, cols // threads, threads), axis=1).reshape(-1)


@pytest.mark.parametrize("threads,loads", [(256, 4), (256, 8), (256, 16), (256, 32), (1024, 4), (1024, 8),
                                           (1024, 16)])
@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (16 * 1000, 3), (16 * 256 * 37, 37),
                                               (16 * 70001, 512)])
def test_read_probe_reads_every_byte(nbytes, workgroups, threads, loads):
    rng = np.random.default_rng(nbytes + workgroups)
    host = rng.integers(0, 256, nbytes + 64, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    sink = torch.full((workgroups * threads,), -1, dtype=torch.int32, device="cuda")
    R.probe_read(src, nbytes, workgroups, sink, threads=threads, loads_in_flight=loads)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, expected_read_fold(host[:nbytes], workgroups, threads))


def test_mfma_probe_matches_the_closed_form():
    # Lane l supplies A row l%32 and B column l%32 with k = 8*(l//32) + e,
    # A = (l%8)/8 + e/16 and B = 1/2 - e/32 (exact in bf16), so every C[m][n]
    # gains sum_k A[m][k] B[k][n] = 2 * sum_e ((m%8)/8 + e/16)(1/2 - e/32) per
    # step.  Lane l's slots 0 and 15 are rows 4*(l//32) and 27 + 4*(l//32); each
    # thread stores 4 chains x (slot 0 + slot 15).  All values are dyadic and
    # small, so the fp32 sums are exact.
    wgs, iters = 3, 8
    sink = torch.zeros(wgs * 512, dtype=torch.float32, device="cuda")
    flops = R.probe_mfma(wgs, iters, sink)
    torch.cuda.synchronize()
    assert flops == wgs * 8 * iters * 4 * 32768

    def step(m):
        return 2.0 * sum(((m % 8) / 8 + e / 16) * (0.5 - e / 32) for e in range(8))

    lane = np.arange(512) % 64
    half = lane // 32
    want = 4 * iters * np.array([step(4 * h) + step(27 + 4 * h) for h in half], dtype=np.float64)
    got = sink.cpu().numpy().reshape(wgs, 512)
    for b in range(wgs):
        np.testing.assert_array_equal(got[b], want.astype(np.float32))
