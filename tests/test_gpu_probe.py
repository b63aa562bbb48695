"""GPU check of the read-stream probe (a measurement aid beside the path):
both load shapes read every byte of the buffer exactly once, so the sum of
the per-block dword sums equals the buffer's dword sum mod 2^32, including
buffers that end inside a 16 KB wave step or a 256-row block."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("pattern", [qm.QMOE_PROBE_LINEAR, qm.QMOE_PROBE_ROWS])
@pytest.mark.parametrize("nbytes", [2048, 16384 + 2048, 3 * (1 << 20) + 6144, 96 << 20])
def test_probe_reads_every_byte_once(pattern, nbytes):
    say(f"stream probe pattern {pattern}, {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes + pattern)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    sink = qm.qmoe_stream_probe(host.to(DEV), pattern).cpu().numpy().view(np.uint32)
    want = int(host.numpy().view(np.uint32).astype(np.uint64).sum()) & 0xFFFFFFFF
    got = int(sink.astype(np.uint64).sum()) & 0xFFFFFFFF
    assert got == want
