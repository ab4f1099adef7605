"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Blobs must be byte-identical to the oracle's, decoded bytes identical to the
input, CRC-32 values identical to zlib's, and corrupted blobs must get the
same verdict (and, when they still decode, the same bytes) as the oracle.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, rans_streams, to_gpu, to_np_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()  # raises if the HIP library is missing
    return m


def gpu_blob(ltc, arr, dtype, chunk=131072, thr=0.95):
    t = to_gpu(arr, dtype)
    return to_np_bytes(ltc.compress(t, chunk, thr))


def gpu_decode(ltc, blob_np):
    b = torch.from_numpy(np.ascontiguousarray(blob_np).copy()).cuda()
    return to_np_bytes(ltc.decompress(b))


def check_case(ltc, arr, dtype, chunk=131072, thr=0.95, label=""):
    banner(f"case {label} dtype={dtype} chunk={chunk} thr={thr} bytes={np.asarray(arr).nbytes}")
    src = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
    want = oracle.compress(src, dtype, chunk, thr)
    got = gpu_blob(ltc, src, dtype, chunk, thr)
    assert got.size == want.size, (got.size, want.size)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"blob differs at {bad.size} bytes, first {bad[:8].tolist()}")
    assert np.array_equal(gpu_decode(ltc, want), src)
    return want


def test_c1_bf16(ltc):
    blob = check_case(ltc, workloads.c1(), 1, label="C1")
    st = ltc.blob_stats(torch.from_numpy(blob))
    assert st["modes"][0]["raw"] == 16 and st["modes"][1]["rans"] == 16


def test_c2_fp32(ltc):
    check_case(ltc, workloads.c2(), 3, label="C2")


def test_c4_clean_fp32_and_fp16(ltc):
    clean, h = workloads.c4()
    check_case(ltc, clean, 3, label="C4 clean fp32")
    check_case(ltc, h, 2, label="C4 fp16")


def _pattern(kind, dtype, nelem, rng):
    e = oracle.ELEM_BYTES[dtype]
    if kind == "normal":
        x = rng.standard_normal(nelem) * 0.02
        if dtype == 0:
            return np.clip(np.rint(x * 2000) + 128, 0, 255).astype(np.uint8)
        if dtype == 1:
            return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
        return x.astype(np.float16 if dtype == 2 else np.float32)
    if kind == "const":
        return np.full(nelem * e, 0x3C, dtype=np.uint8)
    if kind == "two":
        return rng.choice(np.array([0x11, 0xEE], dtype=np.uint8), nelem * e)
    if kind == "random":
        return rng.integers(0, 256, nelem * e, dtype=np.uint8)
    if kind == "special":
        pats = {0: [0, 255, 1], 1: [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x3F80],
                2: [0x0000, 0x8000, 0x7C00, 0xFC00, 0x7E00, 0x0001, 0x3C00],
                3: [0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 1, 0x3F800000]}[dtype]
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[e]
        return rng.choice(np.array(pats, dtype=np.uint64), nelem).astype(dt)
    raise ValueError(kind)


AWKWARD = [(d, n, c, k) for d in (0, 1, 2, 3)
           for n in (0, 1, 63, 64, 65, 129, 1000, 5003, 70001)
           for c in (8, 24, 4096, 131072)
           for k in ("normal", "const", "two", "random", "special")
           if not (c == 8 and n > 5003)]


@pytest.mark.parametrize("dtype,nelem,chunk,kind", AWKWARD,
                         ids=lambda v: str(v))
def test_awkward(ltc, dtype, nelem, chunk, kind):
    rng = np.random.default_rng(nelem * 7 + chunk + dtype)
    arr = _pattern(kind, dtype, nelem, rng)
    check_case(ltc, arr, dtype, chunk, label=f"{kind} n={nelem}")


@pytest.mark.parametrize("thr", [1e-6, 0.3, 0.5, 0.9, 0.95, 1.0])
def test_threshold_variants(ltc, thr):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(300000) * np.repeat([0.02, 0.5, 1e-3], 100000)).astype(np.float32)
    check_case(ltc, x, 3, 65536, thr, label="threshold")
    check_case(ltc, x.astype(np.float16), 2, 65536, thr, label="threshold fp16")


def test_batch_equals_single(ltc):
    rng = np.random.default_rng(8)
    arrs = [(rng.standard_normal(n) * s).astype(np.float32)
            for n, s in ((1, 1.0), (1000, 0.02), (70000, 0.1), (32768, 0.02), (100003, 3.0),
                         (0, 1.0), (262144, 1e-3))]
    ts = [to_gpu(a, 3) for a in arrs]
    blobs = ltc.compress_batch(ts, 65536)
    for a, b in zip(arrs, blobs):
        assert np.array_equal(to_np_bytes(b), oracle.compress(a, 3, 65536))
    outs = ltc.decompress_batch(blobs)
    for a, o in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))


def test_determinism_and_recompress(ltc):
    x = workloads.c1()
    t = to_gpu(x, 1)
    b1 = ltc.compress(t)
    b2 = ltc.compress(t)
    assert torch.equal(b1, b2)
    out = ltc.decompress(b1)
    assert torch.equal(ltc.compress(out), b1)


@pytest.mark.parametrize("n", [0, 1, 100, 4095, 16383, 16384, 16385, 1000007])
@pytest.mark.parametrize("k", [1, 7, 256, 1000, 16384, 65536])
def test_crc32_matches_zlib(ltc, n, k):
    if k == 1 and n > 20000:
        n = 20000
    rng = np.random.default_rng(n + k)
    data = rng.integers(0, 256, n + 3, dtype=np.uint8)
    d = torch.from_numpy(data).cuda()
    for start in (0, 3):  # aligned and misaligned starting address
        view = d[start:start + n]
        got = ltc.crc32_chunks(view, k).cpu().numpy().view(np.uint32).tolist()
        seg = data[start:start + n]
        want = [zlib.crc32(seg[i:i + k].tobytes()) for i in range(0, n, k)]
        assert got == want


def test_crc32_frame_edges(ltc):
    """Chunks whose first bytes sit at the end of a 1 KiB frame of memory (the
    preset's four bytes then cross into the next frame), chunks of 4..17
    bytes, and buffers ending anywhere in a frame."""
    rng = np.random.default_rng(17)
    data = rng.integers(0, 256, 70000, dtype=np.uint8)
    d = torch.from_numpy(data).cuda()
    for start in (509, 510, 511, 1021, 1022, 1023, 1024, 2045):
        for n, k in ((40000, 16384), (3000, 1024), (5000, 1021), (200, 4), (300, 17), (1030, 1027)):
            got = ltc.crc32_chunks(d[start:start + n], k).cpu().numpy().view(np.uint32).tolist()
            seg = data[start:start + n]
            assert got == [zlib.crc32(seg[i:i + k].tobytes()) for i in range(0, n, k)], (start, n, k)


def test_crc32_check_value(ltc):
    d = torch.frombuffer(bytearray(b"123456789"), dtype=torch.uint8).cuda()
    assert ltc.crc32_chunks(d, 16384).cpu().numpy().view(np.uint32).tolist() == [0xCBF43926]


def _verdicts_agree(ltc, blob_np):
    """GPU verdict (host return code or device status) == oracle verdict, and
    identical decoded bytes whenever both accept the blob."""
    want_rc, want = oracle.decompress(blob_np)
    hdr = bytes(blob_np[:64])
    try:
        info = ltc.blob_info(hdr)
    except ltc.LTCError as e:
        assert e.code == want_rc, (e.code, want_rc)
        return want_rc
    b = torch.from_numpy(np.ascontiguousarray(blob_np).copy()).cuda()
    dst = torch.empty(max(1, info["nbytes"]), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    try:
        ltc.decompress_raw([hdr], [b.data_ptr()], [b.numel()], [dst.data_ptr()],
                           [info["nbytes"]], status.data_ptr())
    except ltc.LTCError as e:
        assert e.code == want_rc, (e.code, want_rc)
        return want_rc
    st = int(status.item())
    assert st == want_rc, (st, want_rc)
    if st == 0:
        assert np.array_equal(dst[:info["nbytes"]].cpu().numpy(), want)
    return st


def test_corruption_verdicts_match_oracle(ltc):
    x = workloads.c1()[:200000]
    blob = oracle.compress(x, 1, 16384)
    assert _verdicts_agree(ltc, blob) == 0
    e, k = 2, int.from_bytes(blob[20:24].tobytes(), "little")
    d = blob[64:64 + 16 * k * e].reshape(-1, 16)
    modes = d[:, 12]
    offs = d[:, :8].copy().view(np.uint64).ravel()
    rans = np.nonzero(modes == 1)[0]
    cases = []
    b = blob.copy(); b[64 + 12] = 5; cases.append(("bad mode", b))
    b = blob.copy(); b[64 + 8] ^= 1; cases.append(("size breaks chain", b))
    b = blob.copy(); b[64 + 16 * 3] ^= 0x10; cases.append(("offset breaks chain", b))
    b = blob.copy(); b[64 + 14] = 1; cases.append(("reserved", b))
    o = int(offs[rans[0]])
    b = blob.copy(); b[o + 16 + 2:o + 16 + 4] = 0; cases.append(("state < 2^16", b))
    b = blob.copy(); b[o + 272] ^= 1; cases.append(("table sum", b))
    b = blob.copy(); b[o] ^= 2; cases.append(("word count", b))
    b = blob.copy(); b[o + 6] = 1; cases.append(("prefix zeros", b))
    b = blob.copy(); b[o + 4], b[o + 5] = b[o + 5], b[o + 4]; cases.append(("lo >= hi", b))
    o2 = int(offs[rans[-1]])
    b = blob.copy(); b[o2 + 300] ^= 0x40; cases.append(("word flip", b))
    b = blob.copy(); b[o2 + 16 + 4 * 7] ^= 0x01; cases.append(("state flip", b))
    cases.append(("truncated", blob[:-16]))
    b = blob.copy(); b[4] = 2; cases.append(("version", b))
    b = blob.copy(); b[0] = 0; cases.append(("magic", b))
    for name, cb in cases:
        banner(f"corruption {name}")
        _verdicts_agree(ltc, cb)


def test_random_payload_flips_match_oracle(ltc):
    x = workloads.c1()[:100000]
    blob = oracle.compress(x, 1, 16384)
    base = 64 + 16 * 2 * int.from_bytes(blob[20:24].tobytes(), "little")
    rng = np.random.default_rng(1)
    verdicts = set()
    for i in range(120):
        b = blob.copy()
        pos = int(rng.integers(base, b.size))
        b[pos] ^= 1 << int(rng.integers(0, 8))
        verdicts.add(_verdicts_agree(ltc, b))
    assert -5 in verdicts


def test_crc32_batch_matches_single(ltc):
    rng = np.random.default_rng(3)
    sizes = [0, 1, 16384, 100000, 16384 * 7 + 5, 333]
    ts = [torch.from_numpy(rng.integers(0, 256, n, dtype=np.uint8)).cuda() for n in sizes]
    for k in (16384, 1000):
        outs = ltc.crc32_chunks_batch(ts, k)
        for t, o in zip(ts, outs):
            d = t.cpu().numpy()
            want = [zlib.crc32(d[i:i + k].tobytes()) for i in range(0, d.size, k)]
            assert o.cpu().numpy().view(np.uint32).tolist() == want


@pytest.mark.parametrize("nchunks", [1, 2, 3, 7])
def test_mixed_stream_pairs(ltc, nchunks):
    """Neighbouring chunks alternate between compressible values and random
    bytes (so a wave codes one stream of a pair and not the other), with an
    odd number of chunks as well; blobs must equal the oracle's."""
    rng = np.random.default_rng(nchunks)
    chunk = 16384
    parts = []
    for c in range(nchunks):
        if c % 2 == 0:
            x = (rng.standard_normal(chunk // 2) * 0.02).astype(np.float32)
            parts.append(torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8))
        else:
            parts.append(rng.integers(0, 256, chunk, dtype=np.uint8))
    data = np.concatenate(parts)[: nchunks * chunk - 6]
    check_case(ltc, data, 1, chunk, label=f"mixed pairs {nchunks}")
    check_case(ltc, data[: data.size // 4 * 4], 3, chunk, label=f"mixed pairs fp32 {nchunks}")



def _abandon_mix(dtype, bits, chunk, rng):
    """Chunks whose sign/mantissa bytes are uniform (RAW by the size bound)
    and whose exponent bytes are uniform over 2**bits values: 5 bits code
    well, 7 bits pass the bound but code above P_max, so the encoder
    abandons the exponent stream part way."""
    e_bytes = oracle.ELEM_BYTES[dtype]
    n = chunk // e_bytes
    parts = []
    for b in bits:
        e = rng.integers(0, 1 << b, n) + 40
        if dtype == 1:
            low = rng.integers(0, 256, n)
            parts.append((((low >> 7) << 15) | (e << 7) | (low & 0x7F)).astype(np.uint16))
        else:
            m = rng.integers(0, 1 << 24, n)
            parts.append((((m >> 23) << 31) | (e << 23) | (m & 0x7FFFFF)).astype(np.uint32))
    return np.concatenate(parts)


@pytest.mark.parametrize("dtype", [1, 3])
@pytest.mark.parametrize("thr", [0.88, 0.95])
def test_staged_raw_streams_with_abandoned_neighbours(ltc, dtype, thr):
    """The wave coding a chunk's exponent stream also writes the chunk's RAW
    streams to the workspace for packing; a chunk whose exponent stream is
    abandoned part way, or whose partner's is, packs its RAW streams from
    the input instead.  At threshold 0.88 the 7-bit chunks are abandoned, so
    the chunk pairs cover both abandoned, both coded, and one of each in
    either order (the odd last chunk has no partner); at 0.95 every exponent
    stream is coded.  Blobs must equal the oracle's."""
    rng = np.random.default_rng(31 + dtype)
    x = _abandon_mix(dtype, [7, 7, 5, 5, 7, 5, 5, 7, 5], 131072, rng)
    want = check_case(ltc, x, dtype, 131072, thr, label="abandoned exponent streams")
    e = oracle.ELEM_BYTES[dtype]
    nch = int(want[20:24].view(np.uint32)[0])
    modes = want[64:64 + 16 * nch * e].reshape(nch, e, 16)[:, :, 12]
    assert (modes[:, : e - 1] == 0).all()  # RAW
    top = [0, 0, 1, 1, 0, 1, 1, 0, 1] if thr < 0.9 else [1] * 9  # RAW after abandoning, or RANS
    assert modes[:, e - 1].tolist() == top


# ---- pipelined compression: calls over 4096 chunks or more (the library's
# threshold) run in two chunk-ordered groups on two streams (the caller's and
# one internal stream); blobs must not change.  Chunks of a few thousand
# elements, so that top streams are coded (a RANS payload carries 272 bytes
# of states and its table, more than a stream of 512 bytes may take).

@pytest.mark.parametrize("dtype,chunk", [(1, 8192), (3, 4096), (2, 4096), (0, 2048)])
def test_grouped_single_tensor(ltc, dtype, chunk):
    rng = np.random.default_rng(100 + dtype)
    nbytes = 4200 * chunk + 3 * 8  # 4201 chunks, a ragged last one: two uneven groups (2100 + 2101)
    if dtype == 0:
        data = rng.integers(0, 6, nbytes, dtype=np.uint8)
        data[: nbytes // 3] = 7  # const chunks too
    else:
        x = rng.standard_normal(nbytes // 4) * np.repeat([0.02, 1e-3, 3.0], nbytes // 12 + 1)[: nbytes // 4]
        x = x.astype(np.float32)
        if dtype == 1:
            data = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
            data = np.concatenate([data, data])[:nbytes]
        elif dtype == 2:
            data = np.concatenate([x.astype(np.float16).view(np.uint8)] * 2)[:nbytes]
        else:
            data = x.view(np.uint8)[:nbytes]
        # every 5th chunk random bytes: a RAW and a coded stream in one pair
        for c in range(0, nbytes // chunk, 5):
            data[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    data = data[: nbytes // oracle.ELEM_BYTES[dtype] * oracle.ELEM_BYTES[dtype]]
    want = check_case(ltc, data, dtype, chunk, label=f"grouped dtype {dtype}")
    assert rans_streams(want) > 2000, rans_streams(want)


def test_grouped_batch_with_empty_and_tiny(ltc):
    """A batch whose tensors straddle the group boundaries, with an empty and
    a one-element tensor; every blob must equal the single-tensor oracle blob."""
    rng = np.random.default_rng(77)
    chunk = 4096
    sizes = (720000, 0, 1, 987657, 2, 320000, 2000001, 17, 480000)
    arrs = [(rng.standard_normal(n) * rng.choice([0.02, 1.0, 1e-4])).astype(np.float32) for n in sizes]
    total_chunks = sum((a.nbytes + chunk - 1) // chunk for a in arrs)
    assert total_chunks >= 4096
    ts = [to_gpu(a, 3) for a in arrs]
    banner(f"grouped batch: {len(arrs)} tensors, {total_chunks} chunks")
    blobs = ltc.compress_batch(ts, chunk)
    coded = 0
    for a, b in zip(arrs, blobs):
        want = oracle.compress(a, 3, chunk)
        got = to_np_bytes(b)
        assert got.size == want.size and np.array_equal(got, want)
        coded += rans_streams(want)
    assert coded > 2000, coded
    outs = ltc.decompress_batch(blobs)
    for a, o in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))
    # the same call twice on one stream, and grouped equals a repeat
    again = ltc.compress_batch(ts, chunk)
    for b1, b2 in zip(blobs, again):
        assert torch.equal(b1, b2)


def test_caller_stream_only_equals_grouped(ltc):
    """LTC_FLAG_CALLER_STREAM_ONLY: a call over more than 4096 chunks (which
    otherwise runs in two groups on two streams) runs every kernel on the
    caller's stream and gives the same blobs, plain and with checksums."""
    rng = np.random.default_rng(88)
    chunk = 4096
    arrs = [(rng.standard_normal(n) * s).astype(np.float32) for n, s in
            ((2400000, 0.02), (5, 1.0), (2000003, 1e-3))]
    ts = [to_gpu(a, 3) for a in arrs]
    nbytes = [a.nbytes for a in arrs]
    assert sum((n + chunk - 1) // chunk for n in nbytes) >= 4096
    caps = [ltc.compress_bound(n, 3, chunk) for n in nbytes]
    ws_n = ltc.workspace_size(nbytes, 3, chunk)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    got = {}
    for flags in (0, ltc.FLAG_CALLER_STREAM_ONLY):
        for crc in (0, 16384):
            blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
            sizes = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
            ccap = [(c + 16383) // 16384 for c in caps]
            crcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in ccap]
            ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, 3, chunk, 0.95, flags,
                                [b.data_ptr() for b in blobs], caps, sizes.data_ptr(), ws.data_ptr(), ws_n,
                                crc, [c.data_ptr() for c in crcs] if crc else None, ccap if crc else None)
            torch.cuda.synchronize()
            sz = sizes.cpu().tolist()
            got[(flags, crc)] = ([to_np_bytes(b[:s]) for b, s in zip(blobs, sz)],
                                 [c[:(s + 16383) // 16384].cpu().numpy() for c, s in zip(crcs, sz)] if crc else None)
    coded = 0
    for a, i in zip(arrs, range(len(arrs))):
        want = oracle.compress(a, 3, chunk)
        coded += rans_streams(want)
        for key, (blobs, crcs) in got.items():
            assert np.array_equal(blobs[i], want), (key, i)
            if crcs is not None:
                assert np.array_equal(crcs[i].view(np.uint32), oracle.crc32_chunks(want, 16384)), (key, i)
    assert coded > 2000, coded


@pytest.mark.parametrize("dtype", [0, 1])
def test_largest_chunk_many_histogram_segments(ltc, dtype):
    """chunk_bytes = 16 MiB (the largest): a U8 chunk holds 16 Mi elements and
    a BF16 chunk 8 Mi, so the histogram pass flushes its 16-bit sub-histograms
    many times per chunk; one value dominates (the largest per-copy counts
    a flush allows), and a ragged second chunk follows."""
    rng = np.random.default_rng(900 + dtype)
    chunk = 16 << 20
    nbytes = chunk + 3 * (1 << 20) + 8
    if dtype == 0:
        arr = np.full(nbytes, 7, dtype=np.uint8)
        idx = rng.choice(nbytes, nbytes // 1000, replace=False)
        arr[idx] = rng.integers(0, 256, idx.size, dtype=np.uint8)
    else:
        x = rng.standard_normal(nbytes // 2) * 0.02
        x[: nbytes // 4] = 0.015625  # one bit pattern over half of the first chunk
        arr = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    check_case(ltc, arr, dtype, chunk, label="16 MiB chunks")


@pytest.mark.parametrize("dtype", [0, 1, 3])
@pytest.mark.parametrize("top_last", [False, True], ids=["dir", "top-last"])
def test_wide_and_narrow_symbol_ranges(ltc, dtype, top_last):
    """The encoder keeps a 128-entry table for pairs of streams that span at
    most 128 symbols and a 256-entry one otherwise.  Chunks alternate
    between a narrow coded stream (values 60..75) and a wide one (mostly 5
    and 240, a few in between), so pairs are narrow, wide, and mixed; the
    boundary spans 127, 128 and 129 values appear too."""
    rng = np.random.default_rng(60 + dtype)
    e = oracle.ELEM_BYTES[dtype]
    chunk = 8192
    n = chunk // e
    kinds = ["narrow", "wide", "wide", "narrow", "narrow", "s127", "s128", "s129", "wide"]
    parts = []
    for kind in kinds:
        if kind == "narrow":
            v = rng.integers(60, 76, n)
        elif kind == "wide":
            v = np.where(rng.random(n) < 0.5, 5, 240)
            v[rng.integers(0, n, 40)] = rng.integers(5, 241, 40)
        else:
            span = int(kind[1:])
            v = rng.integers(70, 75, n)
            v[:2] = (10, 10 + span - 1)  # lowest and highest symbol: hi - lo = span - 1
        v = v.astype(np.uint64)
        if dtype == 0:
            parts.append(v.astype(np.uint8))
        elif dtype == 1:  # v is the exponent byte; random sign and mantissa
            low = rng.integers(0, 256, n).astype(np.uint64)
            parts.append((((low >> 7) << 15) | (v << 7) | (low & 0x7F)).astype(np.uint16))
        else:
            m = rng.integers(0, 1 << 24, n).astype(np.uint64)
            parts.append((((m >> 23) << 31) | (v << 23) | (m & 0x7FFFFF)).astype(np.uint32))
    x = np.concatenate(parts)
    src = x.view(np.uint8)
    want = oracle.compress(src, dtype, chunk, top_last=top_last)
    got = to_np_bytes(ltc.compress(to_gpu(src, dtype), chunk, top_last=top_last))
    assert got.size == want.size and np.array_equal(got, want)
    assert np.array_equal(gpu_decode(ltc, want), src)
    st = ltc.blob_stats(torch.from_numpy(want))
    assert st["modes"][e - 1]["rans"] == len(kinds)
