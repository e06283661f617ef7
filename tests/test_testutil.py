"""The test helpers that read the library's 3-bit codec rows (index i in bits 3i .. 3i + 2
of the row as a little-endian bit string), checked by hand cases and a round trip.
No GPU needed."""
import numpy as np

from tests.kvq_testutil import pack3, unpack3


def test_packed3_helpers_round_trip():
    rng = np.random.default_rng(3)
    idx = rng.integers(0, 8, size=(3, 5, 64))
    rows = pack3(idx)
    assert rows.shape == (3, 5, 24)
    assert np.array_equal(unpack3(rows), idx)
    one = np.zeros(16, dtype=np.uint8)
    one[0] = 7                         # bits 0, 1, 2
    one[9] = 5                         # 0b101 at bits 27 .. 29: bits 27 and 29 (byte 3: 8 + 32)
    one[15] = 6                        # 0b110 at bits 45 .. 47: bits 46 and 47 (byte 5: 64 + 128)
    r = pack3(one)
    assert list(r) == [7, 0, 0, 40, 0, 192]
