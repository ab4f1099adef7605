"""GPU parity at the benchmark sizes, in the launch configuration bench.py
times: C3 (28 BF16 tensors, 1.74 GB, one batch call; format v1, the
top-last layout with checksums, format v2 and XOR deltas against the C3D
base) and C5 (one 8 GiB BF16 buffer, 1/8
random bytes) plus CRC-32 of the C5 blob.

Every blob is compared byte for byte with the oracle's blob of the same
input (all 28 C3 tensors in each form, the whole C5 blob), every checksum
with the oracle's CRC-32 of the oracle's blob, and every decode with the
input.  The oracle runs on the host's cores (OpenMP over chunks)."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner

pytestmark = pytest.mark.gpu
CHUNK = 131072
# the oracle's worker threads: the host's CPU share for one GPU
THREADS = max(1, min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))


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


def _host(t):
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy()


def _assert_blob_equal(got, want, what):
    got = got.cpu().numpy() if hasattr(got, "cpu") else got
    assert got.size == want.size, f"{what}: {got.size} bytes against the oracle's {want.size}"
    if not np.array_equal(got, want):
        first = int(np.nonzero(got != want)[0][0])
        raise AssertionError(f"{what}: first differing byte at {first}")


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
    banner(f"C3 oracle parity, all 28 tensors, {THREADS} host threads")
    for i, (t, bl) in enumerate(zip(ts, blobs)):
        want = oracle.compress(_host(t), 1, CHUNK, 0.95, nthreads=THREADS)
        _assert_blob_equal(bl, want, f"C3 tensor {i} {workloads.C3_SHAPES[i]}")
    banner("C3 oracle parity done")


def test_c3_compress_with_crc32_full_size(ltc):
    """compress_with_crc32 over the C3 batch, in bench.py's launch
    configuration: blobs identical to compress_batch, and every checksum
    equal to the oracle's CRC-32 of the blob's chunks."""
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch_with_crc32 (K = 16 KiB)")
    blobs, crcs = ltc.compress_batch_with_crc32(ts, CHUNK, 0.95, 16384)
    plain = ltc.compress_batch(ts)
    for i, (b, p, c) in enumerate(zip(blobs, plain, crcs)):
        assert torch.equal(b, p), i
        ref = ltc.crc32_chunks(b, 16384)
        assert torch.equal(c, ref), i
        want = oracle.crc32_chunks(b.cpu().numpy(), 16384)
        got = c.cpu().numpy().view(np.uint32)
        assert got.size == want.size and np.array_equal(got, want), i
    banner(f"C3 {sum(c.numel() for c in crcs)} checksums equal to the oracle's")


def test_c3_top_last_full_size(ltc):
    """The top-last layout over the C3 batch, as bench.py times it
    (compress_with_crc32, K = 16 KiB, then decompress): all 28 blobs byte
    for byte against the oracle's top-last blobs, every checksum against the
    oracle's CRC-32 of those blobs, the plain call's blobs equal, and the
    exact round trip."""
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch_with_crc32, top-last (K = 16 KiB)")
    blobs, crcs = ltc.compress_batch_with_crc32(ts, CHUNK, 0.95, 16384, top_last=True)
    plain = ltc.compress_batch(ts, top_last=True)
    for i, (b, p) in enumerate(zip(blobs, plain)):
        assert torch.equal(b, p), i
    del plain
    banner("C3 top-last decompress_batch")
    outs = ltc.decompress_batch(blobs)
    for t, o in zip(ts, outs):
        assert torch.equal(t.view(-1).view(torch.int16), o.view(torch.int16))
    del outs
    banner(f"C3 top-last oracle parity, all 28 tensors, {THREADS} host threads")
    for i, (t, bl, c) in enumerate(zip(ts, blobs, crcs)):
        want = oracle.compress(_host(t), 1, CHUNK, 0.95, nthreads=THREADS, top_last=True)
        _assert_blob_equal(bl, want, f"C3 top-last tensor {i} {workloads.C3_SHAPES[i]}")
        wcrc = oracle.crc32_chunks(want, 16384)
        got = c.cpu().numpy().view(np.uint32)
        assert got.size == wcrc.size and np.array_equal(got, wcrc), i
    banner("C3 top-last parity done")


def test_c3_shared_tables_full_size(ltc):
    """Format v2 (one table per stream index) over the C3 batch: exact round
    trip, and all 28 blobs byte for byte against the oracle's v2 blobs."""
    banner("C3 generate")
    ts = workloads.c3_gpu()
    banner("C3 compress_batch, shared tables")
    blobs = ltc.compress_batch(ts, shared_tables=True)
    outs = ltc.decompress_batch(blobs)
    for t, o in zip(ts, outs):
        assert torch.equal(t.view(-1).view(torch.int16), o.view(torch.int16))
    del outs
    banner("C3 v2 oracle parity, all 28 tensors")
    for i, (t, bl) in enumerate(zip(ts, blobs)):
        want = oracle.compress(_host(t), 1, CHUNK, 0.95, nthreads=THREADS, shared_tables=True)
        _assert_blob_equal(bl, want, f"C3 v2 tensor {i} {workloads.C3_SHAPES[i]}")


def test_c3d_delta_full_size(ltc):
    """XOR deltas over the C3D checkpoint pair, as bench.py --delta runs them:
    exact round trip with the bases, and all 28 blobs byte for byte against
    the oracle's delta blobs (tensor 0 is unchanged: CONST streams only)."""
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
    banner("C3D oracle parity, all 28 tensors")
    for i, (f, bs, bl) in enumerate(zip(fine, base, blobs)):
        want = oracle.compress_delta(_host(f), _host(bs), 1, CHUNK, 0.95, nthreads=THREADS)
        _assert_blob_equal(bl, want, f"C3D tensor {i} {workloads.C3_SHAPES[i]}")


@pytest.mark.timeout(600)
def test_c5_full_size_with_crc(ltc):
    """The whole 8 GiB C5 blob against the oracle's, the exact round trip,
    and every CRC-32 chunk of the blob against the oracle's checksums."""
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
    banner(f"C5 ratio {blob.numel() / buf.numel():.4f}")
    banner("C5 GPU CRC-32 of the blob")
    crc = ltc.crc32_chunks(blob, 16384).cpu().numpy().view(np.uint32)
    got = blob.cpu().numpy()
    del blob
    torch.cuda.empty_cache()
    banner("C5 copy the input to the host")
    src = buf.cpu().numpy()
    del buf, t
    torch.cuda.empty_cache()
    banner(f"C5 oracle compress (8 GiB, {THREADS} host threads)")
    want = oracle.compress(src, 1, CHUNK, 0.95, nthreads=THREADS)
    del src
    banner("C5 whole-blob comparison")
    _assert_blob_equal(got, want, "C5 blob")
    del got
    banner("C5 oracle CRC-32 of every 16 KiB chunk")
    wcrc = oracle.crc32_chunks(want, 16384)
    assert crc.size == wcrc.size == (want.size + 16383) // 16384
    bad = np.nonzero(crc != wcrc)[0]
    assert bad.size == 0, f"{bad.size} CRC chunks differ, first {int(bad[0])}"
    banner(f"C5 {crc.size} checksums equal to the oracle's")


def test_c5_top_last_full_size(ltc):
    """C5 as bench.py times it: compress_with_crc32 in the top-last layout
    (65,536 chunks: two streams per encoder wave, payloads placed by the
    encoder, checksums read back), the whole blob against the oracle's
    top-last blob, every checksum against the oracle's CRC-32 of it, and the
    exact round trip."""
    banner("C5 generate (8 GiB)")
    buf = workloads.c5_gpu()
    t = buf.view(torch.bfloat16)
    banner("C5 compress_with_crc32, top-last")
    blob, crc = ltc.compress_with_crc32(t, CHUNK, 0.95, 16384, top_last=True)
    banner("C5 top-last decompress")
    out = ltc.decompress(blob)
    assert torch.equal(out.view(torch.uint8), buf)
    del out
    crc = crc.cpu().numpy().view(np.uint32)
    got = blob.cpu().numpy()
    del blob
    torch.cuda.empty_cache()
    src = buf.cpu().numpy()
    del buf, t
    torch.cuda.empty_cache()
    banner(f"C5 oracle compress, top-last (8 GiB, {THREADS} host threads)")
    want = oracle.compress(src, 1, CHUNK, 0.95, nthreads=THREADS, top_last=True)
    del src
    _assert_blob_equal(got, want, "C5 top-last blob")
    del got
    wcrc = oracle.crc32_chunks(want, 16384)
    assert crc.size == wcrc.size and np.array_equal(crc, wcrc)
    banner(f"C5 top-last: blob and {crc.size} checksums equal to the oracle's")
