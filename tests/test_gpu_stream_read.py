"""The streaming-read measurement aid reads every byte once: the XOR of the
words it writes to its sink equals the XOR of the buffer's 32-bit words."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_util import say  # noqa: E402

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

from block_scaled_fp8_linear_amd import _lib  # noqa: E402


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), (1 << 20, 2048), ((1 << 22) + 48, 7), (3 << 20, 65536)])
def test_stream_read_xor(nbytes, blocks):
    rng = np.random.default_rng(nbytes + blocks)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.full((blocks * 256,), -1, dtype=torch.int32, device="cuda:0")
    say("stream read", nbytes, blocks)
    rc = _lib.stream_read_raw(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0, _lib.status_string(rc)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_binding():
    """The torch-level wrapper: same sink XOR, and a sink too small raises."""
    import block_scaled_fp8_linear_amd as F
    buf = torch.arange(1 << 16, dtype=torch.int32, device="cuda:0")
    sink = F.fp8_block_stream_read(buf, blocks=5)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == \
        np.bitwise_xor.reduce(np.arange(1 << 16, dtype=np.uint32))
    with pytest.raises(ValueError):
        F.fp8_block_stream_read(buf, blocks=5, sink=torch.empty(8, dtype=torch.int32, device="cuda:0"))
