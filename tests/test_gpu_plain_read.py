"""GPU check of qg_plain_read, the measurement utility that reads a buffer
once: every workgroup's sink word is the XOR of exactly its share of the
buffer (so every byte is read once and the ragged end of each share is
covered)."""
import numpy as np
import pytest
import torch

import quantized_weight_decode_dequant_amd as pkg
from helpers import note

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("slots,grid", [(1, 1), (2048, 1), (10007, 7), (2048 * 5 + 17, 3),
                                        (123457, 256)])
def test_plain_read_xor_per_share(slots, grid):
    note("plain read slots=%d grid=%d" % (slots, grid))
    rng = np.random.default_rng(slots)
    words = rng.integers(0, 2**32, size=4 * slots, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    sink = torch.zeros(grid, dtype=torch.int32, device=DEV)
    pkg.qg_plain_read(buf, sink, grid)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    for j in range(grid):
        b0, b1 = j * slots // grid, (j + 1) * slots // grid
        want = np.bitwise_xor.reduce(words[4 * b0:4 * b1]) if b1 > b0 else np.uint32(0)
        assert got[j] == want, "share %d" % j
