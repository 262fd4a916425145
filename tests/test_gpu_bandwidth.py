"""The read-only bandwidth probe (qv_test_read_stream) reads every 16-byte vector of its buffer
exactly once: the XOR of its per-workgroup sinks equals the XOR of the buffer's vectors,
computed on the host, for both access patterns, both cache policies, ragged tails and grids
larger than the work."""
import numpy as np
import pytest

from quantized_weight_verification_amd import _binding as B
from quantized_weight_verification_amd import ops

from _util import dev, host

pytestmark = pytest.mark.gpu


def _xor_vectors(a: np.ndarray) -> np.ndarray:
    return np.bitwise_xor.reduce(a.view(np.int32).reshape(-1, 4), axis=0)


CASES = [
    # (bytes, pattern, row_bytes, blocks)
    (16, B.QV_READ_LINEAR, 0, 1),
    (16 * 1000 + 16 * 7, B.QV_READ_LINEAR, 0, 3),
    (1 << 22, B.QV_READ_LINEAR, 0, 2048),
    ((1 << 22) + 48, B.QV_READ_LINEAR, 0, 97),
    (16 * 64, B.QV_READ_TILES, 64, 1),
    (16 * 4096 * 5, B.QV_READ_TILES, 4096, 2),
    (16 * 4096 * 37, B.QV_READ_TILES, 4096, 2048),
    (16 * 576 * 11, B.QV_READ_TILES, 576, 5),
]


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("nbytes,pattern,row_bytes,blocks", CASES)
def test_read_stream_reads_every_vector_once(nbytes, pattern, row_bytes, blocks, nontemporal):
    rng = np.random.default_rng(nbytes + 7 * blocks + pattern)
    a = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = dev(a)
    sink = ops.read_stream(buf, pattern, row_bytes, nontemporal, blocks)
    got = np.bitwise_xor.reduce(host(sink), axis=0)
    np.testing.assert_array_equal(got, _xor_vectors(a))
