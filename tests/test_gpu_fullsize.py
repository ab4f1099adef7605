"""GPU parity at the benchmark sizes, in the launch configuration bench.py
times: C3 (28 BF16 tensors, 1.74 GB, one batch call) and C5 (one 8 GiB BF16
buffer, 1/8 random bytes) plus CRC-32 of the C5 blob.  Whole outputs are
checked by properties that hold at any size (exact round trip on the GPU,
the directory's offset chain, per-stream modes, determinism); the oracle
recomputes sampled tensors (C3) and sampled chunks (C5) byte for byte; zlib
recomputes sampled CRC chunks."""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner

pytestmark = pytest.mark.gpu
CHUNK = 131072


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _directory(blob):
    info_k = int.from_bytes(blob[20:24].cpu().numpy().tobytes(), "little")
    e = int(blob[7].item())
    d = blob[64:64 + 16 * info_k * e].cpu().numpy().reshape(-1, 16)
    offs = d[:, :8].copy().view(np.uint64).ravel().astype(np.int64)
    sizes = d[:, 8:12].copy().view(np.uint32).ravel().astype(np.int64)
    return e, info_k, offs, sizes, d[:, 12].copy(), d[:, 13].copy()


def _check_chain(blob):
    e, k, offs, sizes, modes, cvals = _directory(blob)
    base = 64 + 16 * k * e
    ends = (offs + sizes + 15) // 16 * 16
    assert offs[0] == base
    assert np.array_equal(offs[1:], ends[:-1])
    assert ends[-1] == blob.numel()
    assert set(np.unique(modes).tolist()) <= {0, 1, 2}
    return e, k, offs, sizes, modes, cvals


def test_c3_batch_full_size(ltc):
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch (28 tensors, one launch sequence)")
    blobs = ltc.compress_batch(ts)
    banner("C3 decompress_batch")
    outs = ltc.decompress_batch(blobs)
    for t, o in zip(ts, outs):
        assert torch.equal(t.view(-1).view(torch.int16), o.view(torch.int16))
    del outs
    n = sum(t.numel() * 2 for t in ts)
    b = sum(x.numel() for x in blobs)
    banner(f"C3 ratio {b / n:.4f}")
    assert 0.64 < b / n < 0.68
    for bl in blobs:
        _, _, _, _, modes, _ = _check_chain(bl)
        assert (modes.reshape(-1, 2)[:, 1] == 1).all()
    assert torch.equal(ltc.compress(ts[2]), blobs[2])      # batch == single call
    assert torch.equal(ltc.compress_batch(ts)[5], blobs[5])  # deterministic
    for i in (0, 1, 4, 27):  # q, k, gate of layer 0 and down of layer 3
        banner(f"C3 oracle parity tensor {i} {workloads.C3_SHAPES[i]}")
        host = ts[i].view(torch.int16).cpu().numpy()
        want = oracle.compress(host, 1, CHUNK, 0.95, nthreads=16)
        assert np.array_equal(blobs[i].cpu().numpy(), want)


def test_c3_compress_with_crc32_full_size(ltc):
    """compress_with_crc32 over the C3 batch, in bench.py's launch
    configuration: blobs identical to compress_batch, checksums identical to
    the CRC kernel's over the finished blobs, sampled chunks equal to zlib."""
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch_with_crc32 (K = 16 KiB)")
    blobs, crcs = ltc.compress_batch_with_crc32(ts, CHUNK, 0.95, 16384)
    plain = ltc.compress_batch(ts)
    rng = np.random.default_rng(5)
    for i, (b, p, c) in enumerate(zip(blobs, plain, crcs)):
        assert torch.equal(b, p), i
        ref = ltc.crc32_chunks(b, 16384)
        assert torch.equal(c, ref), i
        nb = b.numel()
        n = c.numel()
        for w in sorted(set([0, 1, n - 2, n - 1] + rng.integers(0, n, 20).tolist())):
            seg = b[w * 16384:min(nb, (w + 1) * 16384)].cpu().numpy()
            assert int(c[w].item()) & 0xFFFFFFFF == zlib.crc32(seg.tobytes()), (i, w)


def test_c3_shared_tables_full_size(ltc):
    """Format v2 (one table per stream index) over the C3 batch: exact round
    trip, and two tensors byte for byte against the oracle's v2 blobs."""
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch, shared tables")
    blobs = ltc.compress_batch(ts, shared_tables=True)
    outs = ltc.decompress_batch(blobs)
    for t, o in zip(ts, outs):
        assert torch.equal(t.view(-1).view(torch.int16), o.view(torch.int16))
    del outs
    for i in (1, 27):
        banner(f"C3 v2 oracle parity tensor {i} {workloads.C3_SHAPES[i]}")
        host = ts[i].view(torch.int16).cpu().numpy()
        want = oracle.compress(host, 1, CHUNK, 0.95, nthreads=16, shared_tables=True)
        assert np.array_equal(blobs[i].cpu().numpy(), want)


def test_c3d_delta_full_size(ltc):
    """XOR deltas over the C3D checkpoint pair, as bench.py --delta runs them:
    exact round trip with the bases, ZRUN streams present, and three tensors
    byte for byte against the oracle's delta blobs (tensor 0 is unchanged:
    CONST streams only)."""
    banner("C3D generate")
    fine, base = workloads.c3_delta_gpu()
    banner("C3D compress_batch_delta")
    blobs = ltc.compress_batch_delta(fine, base)
    outs = ltc.decompress_batch_delta(blobs, base)
    for t, o in zip(fine, outs):
        assert torch.equal(t.view(-1).view(torch.int16), o.view(torch.int16))
    del outs
    b0 = blobs[0].cpu().numpy()
    k = int.from_bytes(b0[20:24].tobytes(), "little")
    assert b0.size == 64 + 16 * 2 * k and (b0[64 + 12::16] == oracle.MODE_CONST).all()
    zr = sum(sum(m["zrun"] for m in ltc.blob_stats(b)["modes"]) for b in blobs)
    banner(f"C3D ratio {sum(b.numel() for b in blobs) / sum(t.numel() * 2 for t in fine):.4f}, "
           f"{zr} ZRUN streams")
    for i in (1, 6, 27):
        banner(f"C3D oracle parity tensor {i} {workloads.C3_SHAPES[i]}")
        src = fine[i].view(torch.int16).cpu().numpy()
        bs = base[i].view(torch.int16).cpu().numpy()
        want = oracle.compress_delta(src, bs, 1, CHUNK, 0.95, nthreads=16)
        assert np.array_equal(blobs[i].cpu().numpy(), want)


def test_c5_full_size_with_crc(ltc):
    banner("C5 generate (8 GiB)")
    buf = workloads.c5_gpu()
    t = buf.view(torch.bfloat16)
    banner("C5 compress")
    blob = ltc.compress(t)
    banner("C5 decompress")
    out = ltc.decompress(blob)
    assert torch.equal(out.view(torch.uint8), buf)
    del out
    torch.cuda.empty_cache()
    e, k, offs, sizes, modes, cvals = _check_chain(blob)
    assert k == 65536
    m = modes.reshape(k, 2)
    per_tensor = 1024
    rnd = np.zeros(k, dtype=bool)
    for ti in range(7, 64, 8):
        rnd[ti * per_tensor:(ti + 1) * per_tensor] = True
    assert (m[rnd] == 0).all()                 # random bytes: both streams RAW
    assert (m[~rnd, 1] == 1).all() and (m[~rnd, 0] == 0).all()
    ratio = blob.numel() / buf.numel()
    banner(f"C5 ratio {ratio:.4f}")
    rng = np.random.default_rng(0)
    sample = sorted(set([0, 1, 1023, 1024, 7 * 1024, 7 * 1024 + 511, 8 * 1024 - 1, k - 1] +
                        rng.integers(0, k, 40).tolist()))
    for c in sample:
        src = buf[c * CHUNK:(c + 1) * CHUNK].cpu().numpy()
        w_modes, w_cvals, w_sizes, payload = oracle.encode_chunk(src, 1, CHUNK, 0.95, 0)
        assert m[c].tolist() == w_modes.tolist(), c
        assert sizes[2 * c:2 * c + 2].tolist() == w_sizes.tolist(), c
        got = blob[int(offs[2 * c]):int(offs[2 * c]) + payload.size].cpu().numpy()
        assert np.array_equal(got, payload), c
    banner("C5 CRC-32 of the blob")
    crc = ltc.crc32_chunks(blob, 16384).cpu().numpy().view(np.uint32)
    nb = blob.numel()
    assert crc.size == (nb + 16383) // 16384
    idx = sorted(set([0, 1, crc.size - 2, crc.size - 1] + rng.integers(0, crc.size, 2000).tolist()))
    for i in idx:
        lo = i * 16384
        seg = blob[lo:min(nb, lo + 16384)].cpu().numpy()
        assert int(crc[i]) == zlib.crc32(seg.tobytes()), i
