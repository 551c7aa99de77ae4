"""The matrix-core rate probe (a measurement helper, sg_probe.h) runs the
instructions it names: with all-ones operands except one element per lane
group on odd rows (1.125 for e4m3, 2 for int8), every thread's checksum of
two accumulator rows (one even, one odd) after `iters` rounds of 8 chains is
known exactly; the recorded clocks are consistent."""
import numpy as np
import pytest
import torch

import sparse_gemm_layers_amd as sg
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

# per round and chain: an even row sums K values of 1 (one operand is all
# ones), an odd row adds 4 x (1.125 - 1) for e4m3 or 4 x (2 - 1) for int8
EXPECTED = {"mfma_fp8": 8 * (128 + 128.5), "smfmac_fp8": 8 * (64 + 64.5), "mfma_i8": 8 * (64 + 68)}


@pytest.mark.parametrize("kind", list(EXPECTED))
def test_probe_checksum_and_clock(kind):
    iters = 10
    say(f"probe {kind} iters={iters}")
    sink = torch.empty(sg._binding.PROBE_WORKGROUPS * 512, dtype=torch.float32, device=DEV)
    clocks = torch.zeros(4 * sg._binding.PROBE_WORKGROUPS, dtype=torch.int64, device=DEV)
    sg.probe_matrix_rate(kind, iters, sink, clocks)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.all(s == EXPECTED[kind] * iters), (s.min(), s.max())
    c = clocks.cpu().numpy().reshape(-1, 4).astype(np.float64)
    cyc, ticks = c[:, 1] - c[:, 0], c[:, 3] - c[:, 2]
    assert np.all(cyc > 0) and np.all(ticks >= 0)
    ghz = np.median(cyc[ticks > 0] / ticks[ticks > 0]) * 0.1   # real-time counter: 100 MHz
    assert 0.3 < ghz < 3.5, ghz
