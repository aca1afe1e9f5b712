"""The streaming-read ceiling kernel reads every byte once: its per-workgroup
XOR words equal the XOR of the buffer's 32-bit words over each 8 KiB span."""
import numpy as np
import pytest
import torch

from tests import _gpu

pytestmark = pytest.mark.gpu

SPAN = 8192


@pytest.mark.parametrize("nbytes", [16, 4096, SPAN, 3 * SPAN + 48, 40 * SPAN])
def test_stream_read_xor(nbytes):
    qmm = _gpu.lib()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = qmm.qmm_stream_read(src)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    words = SPAN // 4
    want = [np.bitwise_xor.reduce(host[i:i + words]) for i in range(0, host.size, words)]
    assert got.size == len(want) == qmm.qmm_stream_read_sink_words(nbytes)
    assert np.array_equal(got, np.array(want, dtype=np.uint32))


def test_stream_read_rejects_ragged_and_misaligned():
    qmm = _gpu.lib()
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_stream_read(buf[:1000])
    assert e.value.code == -2
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_stream_read(buf[4:4 + 1024])
    assert e.value.code == -7
