"""The measurement probes run and do the work they report: the read probe's
per-block XORs combine to the XOR of every 32-bit word of the buffer, and the
MFMA probe's accumulators all end at 16 x iterations."""
import numpy as np
import pytest
import torch

from tests.gpu_util import host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import probe
else:
    probe = None


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 64 << 20])
def test_stream_read_covers_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    bx = torch.empty(probe.read_blocks(), dtype=torch.int32, device="cuda")
    note(f"probe stream read {nbytes} B")
    probe.stream_read(buf, bx)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(host(bx).view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_mfma_loop_result():
    blocks, iters = 16, 1000
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    note("probe mfma loop")
    probe.mfma(blocks, iters, out)
    torch.cuda.synchronize()
    assert np.all(host(out) == 16.0 * iters)
