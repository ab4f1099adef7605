"""GPU parity of the top-last layout (LTC_FLAG_TOP_LAST; "NOTE-241: ZipNN",
"Method" item 5: the directory maps every payload, so their order is free):
the lower streams' payloads first in directory order, then every chunk's top
stream.  The compressor scans the lower streams before it codes the top
streams, and the wave that codes a chunk's top stream writes the chunk's RAW
streams straight into the blob.

Blobs must equal the oracle's top-last blobs byte for byte, checksums the
oracle's CRC-32 of those blobs, decodes the input, and verdicts on corrupted
blobs the oracle's.  Cases cover every dtype, ragged and tiny inputs, chunks
whose top stream is abandoned part way (so their RAW streams are written
whole by the packing pass instead), calls of 4096 chunks or more (whose
encoder places the top streams' payloads itself; pipelined for deltas, whose
top-stream scans wait on both groups' lower scans), batches with empty
tensors, format v2,
deltas, the fused and the read-back checksums, the per-kernel (event) path
and the host-blob decode.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, rans_streams, to_gpu, to_np_bytes
from test_gpu_parity import _abandon_mix, _pattern

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _events(n):
    import ctypes
    path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
    L = ctypes.CDLL(path)
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    out = []
    for _ in range(n):
        e = ctypes.c_void_p()
        assert L.hipEventCreate(ctypes.byref(e)) == 0
        out.append(e.value)
    return out


def _bytes(arr):
    return np.ascontiguousarray(arr).reshape(-1).view(np.uint8)


def _equal(got, want, what):
    assert got.size == want.size, (what, got.size, want.size)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"{what}: blob differs at {bad.size} bytes, first {bad[:8].tolist()}")


def check(ltc, arr, dtype, chunk=131072, thr=0.95, shared=False, label=""):
    src = _bytes(arr)
    banner(f"top-last {label} dtype={dtype} chunk={chunk} thr={thr} v2={shared} bytes={src.size}")
    want = oracle.compress(src, dtype, chunk, thr, shared_tables=shared, top_last=True)
    got = to_np_bytes(ltc.compress(to_gpu(src, dtype), chunk, thr, shared, top_last=True))
    _equal(got, want, label)
    out = ltc.decompress(torch.from_numpy(want.copy()).cuda())
    assert np.array_equal(to_np_bytes(out), src)
    return want


def test_configs(ltc):
    check(ltc, workloads.c1(), 1, label="C1")
    check(ltc, workloads.c1(), 1, shared=True, label="C1 v2")
    check(ltc, workloads.c2(), 3, label="C2")
    clean, h = workloads.c4()
    check(ltc, clean, 3, label="C4 clean fp32")
    check(ltc, h, 2, label="C4 fp16")


SMALL = [(d, n, c, k) for d in (0, 1, 2, 3)
         for n in (0, 1, 65, 1000, 70001)
         for c in (24, 4096, 131072)
         for k in ("normal", "random", "special")]


@pytest.mark.parametrize("dtype,nelem,chunk,kind", SMALL, ids=lambda v: str(v))
def test_small(ltc, dtype, nelem, chunk, kind):
    rng = np.random.default_rng(nelem * 5 + chunk + dtype)
    check(ltc, _pattern(kind, dtype, nelem, rng), dtype, chunk, label=f"{kind} n={nelem}")


@pytest.mark.parametrize("dtype", [1, 3])
@pytest.mark.parametrize("thr", [0.88, 0.95])
def test_abandoned_top_streams(ltc, dtype, thr):
    """At 0.88 the 7-bit exponent chunks are abandoned part way: their RAW
    streams, partly placed already, are rewritten whole by k_pack."""
    rng = np.random.default_rng(41 + dtype)
    x = _abandon_mix(dtype, [7, 5, 5, 7, 7, 5, 7, 5, 5], 131072, rng)
    check(ltc, x, dtype, 131072, thr, label="abandoned exponent streams")


@pytest.mark.parametrize("dtype,chunk", [(1, 8192), (3, 4096), (2, 4096), (0, 2048)])
def test_grouped_single_tensor(ltc, dtype, chunk):
    """4201 chunks (the library's threshold is 4096): the encoder places the
    top streams' payloads, each after the sizes of the top streams before it
    in the tensor; every fifth chunk is random (a RAW top stream settled
    before coding, inside the sums).  Chunks of a few thousand elements, so
    that the top streams are coded (a RANS payload carries 272 bytes of
    states and its table, more than a stream of 512 bytes may take)."""
    rng = np.random.default_rng(200 + dtype)
    nbytes = 4200 * chunk + 24
    e = oracle.ELEM_BYTES[dtype]
    if dtype == 0:
        data = rng.integers(0, 6, nbytes, dtype=np.uint8)
        data[: nbytes // 3] = 7
    else:
        data = _bytes(_pattern("normal", dtype, nbytes // e, rng))
        data = data.copy()
        for c in range(0, nbytes // chunk, 5):  # random chunks: RAW top streams too
            data[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    want = check(ltc, data[: nbytes // e * e], dtype, chunk, label=f"grouped dtype {dtype}")
    assert rans_streams(want) > 2000, rans_streams(want)


@pytest.mark.parametrize("shared", [False, True], ids=["v1", "v2"])
def test_grouped_batch_with_empty_and_tiny(ltc, shared):
    rng = np.random.default_rng(78)
    chunk = 4096
    sizes = (720000, 0, 1, 987657, 2, 320000, 2000001, 17, 480000)
    arrs = [(rng.standard_normal(n) * rng.choice([0.02, 1.0, 1e-4])).astype(np.float32) for n in sizes]
    assert sum((a.nbytes + chunk - 1) // chunk for a in arrs) >= 4096
    banner(f"top-last grouped batch v2={shared}")
    blobs = ltc.compress_batch([to_gpu(a, 3) for a in arrs], chunk, shared_tables=shared, top_last=True)
    coded = 0
    for i, (a, b) in enumerate(zip(arrs, blobs)):
        want = oracle.compress(a, 3, chunk, shared_tables=shared, top_last=True)
        _equal(to_np_bytes(b), want, f"tensor {i}")
        coded += rans_streams(want)
    assert coded > 2000, coded
    for a, o in zip(arrs, ltc.decompress_batch(blobs)):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))


def test_stream_modes_checksums_and_events(ltc):
    """Calls of 4096 chunks or more (the encoder placing the coded payloads),
    on the caller's stream only or not, and per kernel (events), each plain
    and with checksums of 16 KiB and 1000-byte chunks (in the top-last layout
    the CRC kernel reads the finished blobs back)."""
    rng = np.random.default_rng(89)
    chunk = 4096
    arrs = [(rng.standard_normal(n) * s).astype(np.float32) for n, s in
            ((2400000, 0.02), (5, 1.0), (2000003, 1e-3))]
    ts = [to_gpu(a, 3) for a in arrs]
    nbytes = [a.nbytes for a in arrs]
    caps = [ltc.compress_bound(n, 3, chunk) for n in nbytes]
    ws_n = ltc.workspace_size(nbytes, 3, chunk)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    wants = [oracle.compress(a, 3, chunk, top_last=True) for a in arrs]
    assert sum(rans_streams(w) for w in wants) > 2000
    for flags in (ltc.FLAG_TOP_LAST, ltc.FLAG_TOP_LAST | ltc.FLAG_CALLER_STREAM_ONLY):
        for crc in (0, 16384, 1000):
            for prof in (False, True):
                banner(f"top-last flags={flags} crc={crc} events={prof}")
                blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
                sizes = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
                ccap = [(c + crc - 1) // crc for c in caps] if crc else None
                crcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in ccap] if crc else None
                ev = _events(6 if crc else 5) if prof else None
                ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, 3, chunk, 0.95, flags,
                                    [b.data_ptr() for b in blobs], caps, sizes.data_ptr(), ws.data_ptr(), ws_n,
                                    crc, [c.data_ptr() for c in crcs] if crc else None, ccap, events=ev)
                torch.cuda.synchronize()
                for i, (b, s, want) in enumerate(zip(blobs, sizes.cpu().tolist(), wants)):
                    _equal(to_np_bytes(b[:s]), want, f"tensor {i}")
                    if crc:
                        got = crcs[i][:(s + crc - 1) // crc].cpu().numpy().view(np.uint32)
                        assert np.array_equal(got, oracle.crc32_chunks(want, crc)), (flags, crc, i)


def test_compress_with_crc32_c1(ltc):
    x = workloads.c1()
    want = oracle.compress(x, 1, 131072, top_last=True)
    for k in (1024, 16384, 65536, 7):
        blob, crc = ltc.compress_with_crc32(to_gpu(x, 1), 131072, 0.95, k, top_last=True)
        _equal(to_np_bytes(blob), want, f"C1 K={k}")
        assert np.array_equal(crc.cpu().numpy().view(np.uint32), oracle.crc32_chunks(want, k))


@pytest.mark.parametrize("shared", [False, True], ids=["v1", "v2"])
def test_deltas(ltc, shared):
    rng = np.random.default_rng(12)
    base = workloads.c1()
    src = base.copy()
    idx = rng.integers(0, src.size, src.size // 50)
    src[idx] ^= 1
    want = oracle.compress_delta(src, base, 1, 16384, shared_tables=shared, top_last=True)
    got = ltc.compress_delta(to_gpu(src, 1), to_gpu(base, 1), 16384, shared_tables=shared, top_last=True)
    _equal(to_np_bytes(got), want, f"delta v2={shared}")
    out = ltc.decompress_delta(torch.from_numpy(want.copy()).cuda(), to_gpu(base, 1))
    assert np.array_equal(to_np_bytes(out), _bytes(src))


def test_grouped_deltas_fp32(ltc):
    """Deltas over 4096 chunks run in two groups on two streams: the first
    group's top scan starts where the second group's lower scan ended."""
    rng = np.random.default_rng(13)
    base = (rng.standard_normal(4200 * 256) * 0.02).astype(np.float32)  # 4200 chunks of 1 KiB
    src = base.copy()
    src.view(np.uint32)[rng.integers(0, src.size, 21000)] ^= 3
    want = oracle.compress_delta(src, base, 3, 1024, top_last=True)
    got = ltc.compress_delta(to_gpu(src, 3), to_gpu(base, 3), 1024, top_last=True)
    _equal(to_np_bytes(got), want, "grouped fp32 delta")


def test_host_path(ltc):
    """Oracle top-last blobs decoded from pinned host memory in copy groups
    (two copy ranges per blob and group: lower and top streams)."""
    for arr, dtype, chunk in ((workloads.c2(), 3, 131072), (workloads.c1(), 1, 8192)):
        src = _bytes(arr)
        blob = oracle.compress(src, dtype, chunk, top_last=True)
        h = torch.empty(blob.size, dtype=torch.uint8, pin_memory=True)
        h.numpy()[:] = blob
        banner(f"top-last host decode dtype={dtype} bytes={src.size}")
        out = ltc.decompress_from_host(h)
        assert np.array_equal(to_np_bytes(out), src)
    rng = np.random.default_rng(5)
    arrs = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in (5000000, 0, 3, 2500000)]
    hb = []
    for a in arrs:
        b = oracle.compress(a, 3, 65536, top_last=True)
        h = torch.empty(b.size, dtype=torch.uint8, pin_memory=True)
        h.numpy()[:] = b
        hb.append(h)
    outs = ltc.decompress_batch_from_host(hb)
    for a, o in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))


def test_corruption_verdicts_match_oracle(ltc):
    from test_gpu_parity import _verdicts_agree
    x = workloads.c1()[:200000]
    blob = oracle.compress(x, 1, 16384, top_last=True)
    assert _verdicts_agree(ltc, blob) == 0
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    d = blob[64:64 + 32 * k].reshape(-1, 16)
    offs = d[:, :8].copy().view(np.uint64).ravel()
    cases = []
    b = blob.copy(); b[27] = 0; cases.append(("flag cleared", b))
    v1 = oracle.compress(x, 1, 16384)
    b = v1.copy(); b[27] = 8; cases.append(("flag set on a directory-order blob", b))
    b = blob.copy(); b[64 + 16 * 2] ^= 0x10; cases.append(("lower offset breaks chain", b))
    b = blob.copy(); b[64 + 16 * 3] ^= 0x10; cases.append(("top offset breaks chain", b))
    b = blob.copy(); b[64 + 16 * 1] ^= 0x10; cases.append(("first top offset", b))
    b = blob.copy(); b[64 + 16 * (2 * k - 2) + 8] ^= 1; cases.append(("last lower size", b))
    b = blob.copy(); b[64 + 16 * (2 * k - 1) + 8] ^= 1; cases.append(("last top size", b))
    b = blob.copy()
    b[64 + 16 * 1:64 + 16 * 1 + 8] = np.frombuffer(int(offs[3]).to_bytes(8, "little"), np.uint8)
    b[64 + 16 * 3:64 + 16 * 3 + 8] = np.frombuffer(int(offs[1]).to_bytes(8, "little"), np.uint8)
    cases.append(("top offsets swapped", b))
    cases.append(("truncated", blob[:-16]))
    b = blob.copy(); b[27] |= 16; cases.append(("unknown flag", b))
    for name, cb in cases:
        banner(f"top-last corruption {name}")
        assert _verdicts_agree(ltc, cb) != 0 or name == "none"
    rng = np.random.default_rng(9)
    base = 64 + 32 * k
    for i in range(60):
        b = blob.copy()
        pos = int(rng.integers(base, b.size))
        b[pos] ^= 1 << int(rng.integers(0, 8))
        _verdicts_agree(ltc, b)
