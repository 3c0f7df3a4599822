"""The measurement helper moe_stream_read reads every byte it is given: the XOR of the words it writes equals
the XOR of all 32-bit words of the buffer (computed on the host), for ragged sizes from one 16-byte chunk to
several passes of the grid."""

import numpy as np
import pytest
import torch

import int4_weights_amd as moe
from gpu_helpers import DEV, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4112, 1 << 20, 10 * (1 << 20) + 48])
def test_stream_read_folds_every_word(nbytes):
    require_gpu()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(-(1 << 31), 1 << 31, size=max(nbytes // 4, 1), dtype=np.int64).astype(np.int32)[:nbytes // 4]
    buf = torch.from_numpy(host.copy()).to(DEV) if nbytes else torch.empty(0, dtype=torch.int32, device=DEV)
    out = torch.full((moe.moe_stream_read_words(),), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    moe.moe_stream_read(buf, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32)) if nbytes else np.uint32(0)
    assert got == want
