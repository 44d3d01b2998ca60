"""The streaming-read yardstick (qhead_stream_read): every 32-bit word of the
buffer is read exactly once, so the XOR of its per-workgroup words equals
numpy's XOR over the same words, for sizes from one 16-byte vector to several waves' worth with a
ragged tail, and for a buffer larger than one pass of the whole grid."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_weight_decode_amd as qh
    return qh


@pytest.mark.parametrize("nbytes", [16, 1024, 4096 + 16, 3 * 2**20 + 48, 96 * 2**20 + 4080])
def test_stream_read_xor_matches_numpy(qh, nbytes):
    print(f"stream_read bytes={nbytes}", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    words = qh.stream_read(buf).cpu().numpy().view(np.uint32)
    got = np.bitwise_xor.reduce(words)
    want = np.bitwise_xor.reduce(host)
    assert got == want


def test_stream_read_twice_same_output_tensor(qh):
    """The output word is cleared by the binding before each call."""
    host = np.arange(1, 4097, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((qh.STREAM_READ_WORDS,), 12345, dtype=torch.int32, device="cuda")
    for _ in range(2):
        words = qh.stream_read(buf, xor_out=out).cpu().numpy().view(np.uint32)
        assert np.bitwise_xor.reduce(words) == np.bitwise_xor.reduce(host)
