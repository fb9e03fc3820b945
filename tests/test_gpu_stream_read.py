"""The plain streaming read that prices the fused kernel's HBM ceiling: what it
folds must be every byte of the buffer, whatever the size (a workgroup per
compute unit, ragged tails, workgroups with nothing to read)."""
import numpy as np
import pytest
import torch

import decode_exact_categorical_amd as fs
from gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def xor_fold(buf: np.ndarray) -> int:
    """The kernel's fold: the xor of the buffer's 16-byte pieces, then of its
    first and third 32-bit words (high half) and second and fourth (low half)."""
    x = np.bitwise_xor.reduce(buf.view(np.uint32).reshape(-1, 4), axis=0)
    return (int(x[0] ^ x[2]) << 32) | int(x[1] ^ x[3])


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 255, 16 * 257, (1 << 20) + 16, (64 << 20) + 48])
def test_stream_read_folds_every_byte(dev, nbytes):
    say(f"stream read of {nbytes} bytes")
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).to(dev)
    out = fs.debug_stream_read(buf)
    torch.cuda.synchronize()
    got = int(out.cpu().numpy().view(np.uint64)[0])
    assert got == xor_fold(host)
    # A second call folds into the same word: the two cancel.
    fs.debug_stream_read(buf, out)
    torch.cuda.synchronize()
    assert int(out.cpu()[0]) == 0
