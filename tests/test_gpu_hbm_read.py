"""GPU check of the read-ceiling helper (lowbit_hbm_read) through the C ABI:
it reads every 16-byte block once and each workgroup stores the XOR of the
32-bit words it read to its own sink word, so the XOR over the sink is
compared bit for bit with numpy's XOR reduction of the same bytes (sizes: one
block, ragged chunk tails, chunks of several 16 KiB rounds per wave).  The
sink starts filled with a pattern: every word must be written."""
import numpy as np
import pytest
import torch

import bit_weight_only_pack_amd as lb
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * 257, 16 * 4096 * 3 + 48, 16 * (4096 * 1024 * 2 + 777)])
def test_hbm_read_xor_matches_numpy(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = dev(host.view(np.int32))
    sink = torch.full((lb.LOWBIT_HBM_READ_SINK_WORDS,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    lb.check(lb.lowbit_hbm_read(buf, nbytes, sink))
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
