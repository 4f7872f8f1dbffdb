"""The read-stream probe (benchmark only) reads every 32-bit word of its
buffer exactly once in every variant: the xor of all its output words equals
the xor of the buffer's words (a word read twice would cancel, a word missed
would be absent).  The buffer size leaves a ragged tail for every grid."""
import numpy as np
import pytest
import torch

import quant_weight_matvec_amd as kq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("unroll", [1, 4, 8, 16])
@pytest.mark.parametrize("flags", [0, 1, 2, 3])
@pytest.mark.parametrize("grid,block", [(7, 64), (256, 256), (1024, 512), (300, 1024)])
def test_probe_reads_every_word_once(unroll, flags, grid, block):
    rng = np.random.default_rng(unroll * 100 + flags * 10 + grid)
    n16 = 777_777  # 16-byte pieces
    host = rng.integers(0, 2**31, size=4 * n16, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    out = torch.zeros(grid * block // 64, dtype=torch.int32, device="cuda")
    kq.kq_probe_read_bw(buf, 16 * n16, out, grid, block, unroll, flags)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want
