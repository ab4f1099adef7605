"""Pins for the oracle's per-chunk CRC-32: the published check value and
Python's zlib.crc32 (cuZipNN's checksums are defined to match zlib)."""
import zlib

import numpy as np
import pytest

import oracle


def test_check_value():
    assert oracle.crc32(np.frombuffer(b"123456789", dtype=np.uint8)) == 0xCBF43926


@pytest.mark.parametrize("n,k", [(0, 16384), (1, 16384), (16383, 16384), (16384, 16384),
                                 (16385, 16384), (100000, 16384), (100000, 1), (1000, 7),
                                 (70001, 256)])
def test_chunks_match_zlib(n, k):
    rng = np.random.default_rng(n + k)
    data = rng.integers(0, 256, n).astype(np.uint8)
    got = oracle.crc32_chunks(data, k)
    want = [zlib.crc32(data[i:i + k].tobytes()) for i in range(0, n, k)]
    assert got.tolist() == want
