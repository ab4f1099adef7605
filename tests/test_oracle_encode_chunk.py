"""Pin of the oracle's per-chunk entry point (ltco_encode_chunk) against its
whole-blob compress (ltco_compress, pinned by the hand-built blobs, the rANS
goldens and the round trips).

The full-size GPU test of the 8 GiB workload may use encode_chunk to look at
single chunks, so its output must be exactly the chunk's bytes of the blob:
for every chunk c, the E payloads it returns, each zero-padded to 16 and
concatenated, sit at the directory offset of stream c*E in compress's blob,
and its modes, constant values and sizes are the directory's fields (the
cursor rule of the blob format: payloads follow each other in directory
order at 16-byte aligned offsets, gaps zero)."""
import numpy as np
import pytest

import oracle
import workloads


def _dir(blob):
    e = int(blob[7])
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    d = blob[64:64 + 16 * k * e].reshape(-1, 16)
    offs = d[:, :8].copy().view(np.uint64).ravel().astype(np.int64)
    sizes = d[:, 8:12].copy().view(np.uint32).ravel()
    return e, k, offs, sizes, d[:, 12].copy(), d[:, 13].copy()


def _check_every_chunk(x, dtype, chunk_bytes, threshold=0.95):
    blob = oracle.compress(x, dtype, chunk_bytes, threshold, nthreads=4)
    e, k, offs, sizes, modes, cvals = _dir(blob)
    seen_modes = set()
    for c in range(k):
        m, cv, sz, payload = oracle.encode_chunk(x, dtype, chunk_bytes, threshold, c)
        sl = slice(c * e, (c + 1) * e)
        assert m.tolist() == modes[sl].tolist(), c
        assert cv.tolist() == cvals[sl].tolist(), c
        assert sz.tolist() == sizes[sl].tolist(), c
        # the chunk's payload region runs from its first stream's offset to
        # the next chunk's first offset (or the blob's end)
        start = int(offs[c * e])
        end = int(offs[(c + 1) * e]) if c + 1 < k else blob.size
        assert payload.size == end - start, c
        assert np.array_equal(payload, blob[start:end]), c
        seen_modes |= set(m.tolist())
    return seen_modes


def test_every_chunk_of_c1():
    """16 chunks of BF16: RAW sign/mantissa streams and RANS exponents."""
    assert _check_every_chunk(workloads.c1(), 1, 131072) == {oracle.MODE_RAW, oracle.MODE_RANS}


def test_every_chunk_ragged_fp32_with_constant_bytes():
    """FP32 with a ragged last chunk: clean values (two CONST low bytes),
    noisy values (RAW) and a constant run, at a small chunk size so the
    input spans many chunks."""
    rng = np.random.default_rng(11)
    clean = (rng.standard_normal(3000) * 0.02).astype(np.float32)
    clean = (clean.view(np.uint32) & 0xFFFF0000).view(np.float32)
    noisy = (rng.standard_normal(2500) * 0.5).astype(np.float32)
    flat = np.full(1100, 1.5, dtype=np.float32)
    x = np.concatenate([clean, noisy, flat, noisy[:333]])
    assert x.nbytes % 4096 != 0
    seen = _check_every_chunk(x, 3, 4096)
    assert seen == {oracle.MODE_RAW, oracle.MODE_RANS, oracle.MODE_CONST}


def test_every_chunk_ragged_u8():
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.integers(0, 4, 5000), np.zeros(5000, dtype=np.int64),
                        rng.integers(0, 256, 4000), rng.integers(100, 103, 777)]).astype(np.uint8)
    seen = _check_every_chunk(x, 0, 2048)
    assert seen == {oracle.MODE_RAW, oracle.MODE_RANS, oracle.MODE_CONST}


@pytest.mark.parametrize("chunk", [0, 3])
def test_encode_chunk_rejects_out_of_range(chunk):
    x = workloads.c1()[:3 * 65536 // 2]  # 1.5 chunks
    if chunk == 0:
        oracle.encode_chunk(x, 1, 131072, 0.95, 0)
        return
    with pytest.raises(ValueError):
        oracle.encode_chunk(x, 1, 131072, 0.95, chunk)
