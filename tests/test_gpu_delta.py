"""GPU parity of XOR deltas ("NOTE-241: ZipNN", Method item 6 and the Deltas
results: the XOR of two checkpoints, with ZipNN's rule choosing a zero-run
coder for byte groups that are mostly zero bytes).  Delta blobs written by
the HIP path must equal the oracle's byte for byte (format v1 and v2), the
oracle's delta blobs must decode on the GPU to the input given the base, and
corrupted zero-run payloads must get the oracle's verdict.  Inputs cover every
dtype, ragged and one-element tensors, identical tensors (CONST only), sparse
and dense changes, unchanged runs, misaligned bases, batches split into chunk
groups on several streams, and checksums read back from delta blobs.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import banner, stream_modes, to_gpu, to_np_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def _modes(blob):
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    e = int(blob[7])
    return blob[64 + 12:64 + 16 * k * e:16]


def check_delta(ltc, src, base, dtype, chunk=131072, thr=0.95, shared=False, label="", top_last=False):
    sb = np.ascontiguousarray(src).reshape(-1).view(np.uint8)
    bb = np.ascontiguousarray(base).reshape(-1).view(np.uint8)
    banner(f"delta case {label} dtype={dtype} chunk={chunk} thr={thr} v2={shared} top_last={top_last} "
           f"bytes={sb.size}")
    want = oracle.compress_delta(sb, bb, dtype, chunk, thr, shared_tables=shared, top_last=top_last)
    tb = to_gpu(bb, dtype)
    got = to_np_bytes(ltc.compress_delta(to_gpu(sb, dtype), tb, chunk, thr, shared_tables=shared,
                                         top_last=top_last))
    assert got.size == want.size, (got.size, want.size)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"delta blob differs at {bad.size} bytes, first {bad[:8].tolist()}")
    out = ltc.decompress_delta(torch.from_numpy(want.copy()).cuda(), tb)
    assert np.array_equal(to_np_bytes(out), sb)
    return want


def _pair(dtype, nelem, kind, rng):
    """(src, base) element arrays of one of the delta kinds."""
    e = oracle.ELEM_BYTES[dtype]
    x = rng.standard_normal(nelem) * 0.02
    if dtype == 0:
        base = np.clip(np.rint(x * 2000) + 128, 0, 255).astype(np.uint8)
    elif dtype == 1:
        base = _bf16(x).view(np.uint16)
    else:
        base = x.astype(np.float16 if dtype == 2 else np.float32).view(np.uint16 if dtype == 2 else np.uint32)
    src = base.copy()
    if kind == "identical":
        pass
    elif kind == "nudge":  # 10% of the elements move by a few units in the last place
        idx = rng.choice(nelem, nelem // 10, replace=False) if nelem else np.zeros(0, np.int64)
        src[idx] = (src[idx].astype(np.int64) + rng.integers(-3, 4, idx.size)).astype(src.dtype)
    elif kind == "sparse":  # 0.5% change anywhere in the element
        idx = rng.choice(nelem, max(1, nelem // 200), replace=False) if nelem else np.zeros(0, np.int64)
        src[idx] = rng.integers(0, 1 << (8 * e), idx.size, dtype=np.uint64).astype(src.dtype)
    elif kind == "runs":  # unchanged runs, then a dense change
        for c0 in range(0, nelem, 4096):
            hi = min(nelem, c0 + 4096)
            lo = c0 + (hi - c0) * 3 // 4
            src[lo:hi] = rng.integers(0, 1 << (8 * e), hi - lo, dtype=np.uint64).astype(src.dtype)
    elif kind == "random":
        src = rng.integers(0, 1 << (8 * e), nelem, dtype=np.uint64).astype(src.dtype)
    return src, base


def test_c1_nudged(ltc):
    rng = np.random.default_rng(1)
    x = workloads.c1()
    y = x.copy()
    idx = rng.choice(y.size, y.size // 10, replace=False)
    y[idx] = (y[idx].astype(np.int32) + rng.integers(-3, 4, idx.size)).astype(y.dtype)
    blob = check_delta(ltc, y, x, 1, label="C1 nudged")
    assert ltc.blob_info(bytes(blob[:64]))["flags"] == oracle.FLAG_DELTA
    # scattered one-ulp changes: the XOR's exponent byte is almost all zero
    # bytes, yet spread so thinly that rANS beats the run coder
    modes = _modes(blob).reshape(-1, 2)
    assert (modes[:, 1] == oracle.MODE_RANS).all()
    st = ltc.blob_stats(torch.from_numpy(blob.copy()).cuda())
    assert [m["rans"] for m in st["modes"]] == [int((modes[:, q] == oracle.MODE_RANS).sum()) for q in (0, 1)]
    assert sum(m["zrun"] for m in st["modes"]) == int((modes == oracle.MODE_ZRUN).sum())
    check_delta(ltc, y, x, 1, shared=True, label="C1 nudged v2")


KINDS = ("identical", "nudge", "sparse", "runs", "random")
SMALL = [(d, n, c, k) for d in (0, 1, 2, 3) for n in (0, 1, 63, 1000, 5003, 70001)
         for c in (8, 24, 4096, 131072) for k in KINDS if not (c == 8 and n > 5003)]


@pytest.mark.parametrize("dtype,nelem,chunk,kind", SMALL, ids=lambda v: str(v))
def test_small(ltc, dtype, nelem, chunk, kind):
    rng = np.random.default_rng(nelem * 13 + chunk + dtype)
    src, base = _pair(dtype, nelem, kind, rng)
    check_delta(ltc, src, base, dtype, chunk, label=f"{kind} n={nelem}")
    if chunk in (24, 4096):
        check_delta(ltc, src, base, dtype, chunk, shared=True, label=f"{kind} n={nelem}")


@pytest.mark.parametrize("thr", [1e-6, 0.5, 0.95, 1.0])
def test_thresholds(ltc, thr):
    rng = np.random.default_rng(8)
    src, base = _pair(3, 300_000, "nudge", rng)
    check_delta(ltc, src, base, 3, 65536, thr, label="threshold")
    src, base = _pair(1, 300_000, "runs", rng)
    check_delta(ltc, src, base, 1, 65536, thr, label="threshold runs")


def test_oracle_cases_both_coders(ltc):
    """Unchanged runs (ZRUN and CONST) and FP32 nudges (ZRUN, CONST and RANS
    streams side by side in one blob)."""
    rng = np.random.default_rng(21)
    x = workloads.c1()[:300_000]
    z = x.copy()
    for c0 in range(0, z.size, 32768):
        z[c0 + 24000:c0 + 32768] = rng.integers(0, 65536, z[c0 + 24000:c0 + 32768].size).astype(z.dtype)
    f, g = _pair(3, 300_000, "nudge", np.random.default_rng(3))
    for shared in (False, True):
        blob = check_delta(ltc, z, x, 1, 65536, shared=shared, label="unchanged runs")
        assert set(_modes(blob).tolist()) == {oracle.MODE_ZRUN, oracle.MODE_CONST}
        blob = check_delta(ltc, f, g, 3, 65536, shared=shared, label="fp32 nudges")
        assert set(_modes(blob).tolist()) == {oracle.MODE_ZRUN, oracle.MODE_CONST, oracle.MODE_RANS}


@pytest.mark.parametrize("dtype", [1, 3])
def test_staged_raw_xor_streams(ltc, dtype):
    """Every mantissa bit changes at random while 30% of the exponents move by
    one: the XOR's mantissa streams are RAW and its exponent stream is coded,
    so the encoder stages the RAW XOR bytes for packing (all chunk pairs but
    the odd last chunk).  Blobs must equal the oracle's."""
    rng = np.random.default_rng(40 + dtype)
    e = oracle.ELEM_BYTES[dtype]
    n = 9 * 131072 // e
    _, base = _pair(dtype, n, "identical", rng)
    wm = 7 if dtype == 1 else 23  # mantissa width
    mant = rng.integers(0, 1 << wm, n, dtype=np.uint64)
    sign = rng.integers(0, 2, n, dtype=np.uint64) << (8 * e - 1)
    bump = (rng.random(n) < 0.3).astype(np.uint64) << wm  # exponent +1 (a carry into it)
    b64 = base.astype(np.uint64)
    src = (((b64 & ~np.uint64((1 << wm) - 1)) + bump) ^ sign | mant) & np.uint64((1 << (8 * e)) - 1)
    src = src.astype(base.dtype)
    blob = check_delta(ltc, src, base, dtype, label="staged RAW XOR streams")
    modes = _modes(blob).reshape(-1, e)
    assert (modes[:, : e - 1] == oracle.MODE_RAW).all()
    assert (modes[:, e - 1] == oracle.MODE_RANS).all()


@pytest.mark.parametrize("dtype,chunk,shared", [(1, 1024, False), (1, 1024, True), (3, 512, False),
                                                (0, 512, True)])
def test_grouped(ltc, dtype, chunk, shared):
    """Over 4096 chunks: two chunk groups on two streams (v2: after the
    tables), ZRUN chunks in every group."""
    rng = np.random.default_rng(500 + dtype)
    e = oracle.ELEM_BYTES[dtype]
    n = (4200 * chunk + 24) // e
    src, base = _pair(dtype, n, "nudge", rng)
    sv = src.view(np.uint8)
    for c in range(0, sv.size // chunk, 7):  # some chunks changed everywhere
        sv[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    check_delta(ltc, src, base, dtype, chunk, shared=shared, label=f"grouped {dtype}")


@pytest.mark.parametrize("top_last", [False, True], ids=["dir", "top-last"])
def test_two_streams_per_wave(ltc, top_last):
    """33,000 chunks: each pipeline group holds 16,384 chunks or more, so the
    encoder codes two chunks' streams per wave (the workgroups of a chunk pair
    8 apart for the XCDs), with ZRUN, RANS and RAW streams in every group.
    8 KiB chunks (2048 elements per stream), so that a RANS payload fits: every
    fifth chunk XORs small nonzero values into its low bytes (no zero runs,
    three bits a symbol), every eleventh is random bytes."""
    rng = np.random.default_rng(530)
    chunk = 8192
    n = (33000 * chunk) // 4
    src, base = _pair(3, n, "nudge", rng)
    per = chunk // 4
    for c in range(2, n // per, 5):
        src[c * per:(c + 1) * per] = base[c * per:(c + 1) * per] ^ rng.integers(1, 8, per, dtype=np.uint32)
    sv = src.view(np.uint8)
    for c in range(0, sv.size // chunk, 11):
        sv[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    want = check_delta(ltc, src, base, 3, chunk, top_last=top_last, label="two streams per wave")
    modes = stream_modes(want)
    for half in (modes[: modes.shape[0] // 2], modes[modes.shape[0] // 2:]):
        counts = np.bincount(half.reshape(-1), minlength=4)
        assert counts[0] > 0 and counts[1] > 1000 and counts[3] > 1000, counts  # RAW, RANS, ZRUN


def test_misaligned_base_and_source(ltc):
    """Bases and sources aligned to the element only (the scalar load path)."""
    rng = np.random.default_rng(33)
    for dtype, kind in ((1, "nudge"), (3, "runs"), (2, "sparse")):
        src, base = _pair(dtype, 90_001, kind, rng)
        e = oracle.ELEM_BYTES[dtype]
        want = oracle.compress_delta(src, base, dtype, 16384)
        tdt = {1: torch.bfloat16, 2: torch.float16, 3: torch.float32}[dtype]
        for so, bo in ((0, 1), (1, 0), (3, 5)):
            sbuf = torch.zeros(src.size + 8, dtype=tdt, device="cuda")
            bbuf = torch.zeros(base.size + 8, dtype=tdt, device="cuda")
            ts, tb = sbuf[so:so + src.size], bbuf[bo:bo + base.size]
            ts.view(torch.uint8).copy_(torch.from_numpy(src.view(np.uint8).copy()).cuda())
            tb.view(torch.uint8).copy_(torch.from_numpy(base.view(np.uint8).copy()).cuda())
            assert (ts.data_ptr() % 16 != 0) or (tb.data_ptr() % 16 != 0) or so == bo == 0
            banner(f"misaligned dtype={dtype} offsets=({so * e},{bo * e})")
            got = to_np_bytes(ltc.compress_delta(ts, tb, 16384))
            assert np.array_equal(got, want), (dtype, so, bo)
            out = ltc.decompress_delta(torch.from_numpy(want.copy()).cuda(), tb)
            assert np.array_equal(to_np_bytes(out), src.view(np.uint8))


def test_batch_with_empty_and_tiny(ltc):
    rng = np.random.default_rng(79)
    chunk = 1024
    sizes = (90000, 0, 1, 123457, 2, 40000, 250001, 17, 60000)
    kinds = ("nudge", "identical", "random", "runs", "sparse", "nudge", "runs", "identical", "random")
    pairs = [_pair(3, n, k, rng) for n, k in zip(sizes, kinds)]
    for shared in (False, True):
        banner(f"delta batch v2={shared}")
        ts = [to_gpu(s, 3) for s, _ in pairs]
        bs = [to_gpu(b, 3) for _, b in pairs]
        blobs = ltc.compress_batch_delta(ts, bs, chunk, shared_tables=shared)
        for (s, b), bl in zip(pairs, blobs):
            assert np.array_equal(to_np_bytes(bl), oracle.compress_delta(s, b, 3, chunk, shared_tables=shared))
        outs = ltc.decompress_batch_delta(blobs, bs)
        for (s, _), o in zip(pairs, outs):
            assert np.array_equal(to_np_bytes(o), s.view(np.uint8))


def test_checksums_read_back(ltc):
    """ltc_compress_batch_ex with bases and checksums: the CRC kernel reads
    the finished delta blobs back; CRC-32 per 16 KiB equals zlib's."""
    rng = np.random.default_rng(44)
    pairs = [_pair(1, n, k, rng) for n, k in ((3_000_000, "nudge"), (70_001, "runs"), (0, "identical"))]
    ts = [to_gpu(s, 1) for s, _ in pairs]
    bs = [to_gpu(b, 1) for _, b in pairs]
    nbytes = [t.numel() * 2 for t in ts]
    caps = [ltc.compress_bound(n, 1) for n in nbytes]
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    ccaps = [(c + 16383) // 16384 for c in caps]
    crcs = [torch.empty(c, dtype=torch.int32, device="cuda") for c in ccaps]
    ws = torch.empty(max(ltc.workspace_size(nbytes, 1), 256), dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
    ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, 1, 131072, 0.95, 0, [b.data_ptr() for b in blobs],
                        caps, sizes.data_ptr(), ws.data_ptr(), ws.numel(), 16384,
                        [c.data_ptr() for c in crcs], ccaps, base_ptrs=[b.data_ptr() for b in bs])
    for (s, b), bl, c, n in zip(pairs, blobs, crcs, sizes.cpu().tolist()):
        want = oracle.compress_delta(s, b, 1)
        assert n == want.size and np.array_equal(bl[:n].cpu().numpy(), want)
        got = c[:(n + 16383) // 16384].cpu().numpy().view(np.uint32).tolist()
        assert got == [zlib.crc32(want[i:i + 16384].tobytes()) for i in range(0, n, 16384)]


def test_base_rules_and_errors(ltc):
    x = workloads.c1()[:100_000]
    y = x.copy()
    y[::50] ^= 1
    tx, ty = to_gpu(x, 1), to_gpu(y, 1)
    dblob = ltc.compress_delta(ty, tx)
    plain = ltc.compress(ty)
    with pytest.raises(ltc.LTCError) as e:  # a delta blob needs its base
        ltc.decompress(dblob)
    assert e.value.code == -1
    with pytest.raises(ltc.LTCError) as e:  # a plain blob takes none
        ltc.decompress_delta(plain, tx)
    assert e.value.code == -1
    with pytest.raises(ltc.LTCError) as e:  # the host-blob path decodes plain blobs only
        ltc.decompress_from_host(dblob.cpu())
    assert e.value.code == -1
    hdr = bytes(dblob[:64].cpu().numpy().tobytes())
    need = ltc.delta_workspace_size([hdr])
    assert need == x.size * 2 // 131072 * 131072 + (131072 if x.size * 2 % 131072 else 0)
    # slots are 16-byte aligned: C = 24 bytes of FP32 holds 6 elements, slot 16
    h24 = bytes(oracle.compress_delta(x[:1000], x[:1000], 3, 24)[:64])
    assert ltc.delta_workspace_size([h24]) == (2000 + 23) // 24 * 4 * 16
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    dst = torch.empty(x.size * 2, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    with pytest.raises(ltc.LTCError) as e:  # workspace one byte short
        ltc.decompress_delta_raw([hdr], [dblob.data_ptr()], [dblob.numel()], [tx.data_ptr()],
                                 [dst.data_ptr()], [dst.numel()], status.data_ptr(), ws.data_ptr(), need - 1)
    assert e.value.code == -7
    with pytest.raises(ltc.LTCError) as e:  # misaligned base
        ltc.decompress_delta_raw([hdr], [dblob.data_ptr()], [dblob.numel()], [tx.data_ptr() + 1],
                                 [dst.data_ptr()], [dst.numel()], status.data_ptr(), ws.data_ptr(), need)
    assert e.value.code == -1
    ltc.decompress_delta_raw([hdr], [dblob.data_ptr()], [dblob.numel()], [tx.data_ptr()],
                             [dst.data_ptr()], [dst.numel()], status.data_ptr(), ws.data_ptr(), need)
    assert int(status.item()) == 0 and torch.equal(dst, ty.view(torch.uint8))
    # identical tensors: CONST streams only, no payload bytes
    same = to_np_bytes(ltc.compress_delta(tx, tx))
    assert (_modes(same) == oracle.MODE_CONST).all() and same.size == 64 + 16 * _modes(same).size


def test_corrupt_zrun_payloads_match_oracle_verdicts(ltc):
    rng = np.random.default_rng(4)
    x = workloads.c1()[:200_000]
    z = x.copy()
    for c0 in range(0, z.size, 32768):
        z[c0 + 24000:c0 + 32768] = rng.integers(0, 65536, z[c0 + 24000:c0 + 32768].size).astype(z.dtype)
    tx = to_gpu(x, 1)
    for shared in (False, True):
        blob = oracle.compress_delta(z, x, 1, 65536, shared_tables=shared)
        k = int.from_bytes(blob[20:24].tobytes(), "little")
        ents = [(int.from_bytes(blob[64 + 16 * i:72 + 16 * i].tobytes(), "little"),
                 int.from_bytes(blob[72 + 16 * i:76 + 16 * i].tobytes(), "little"), int(blob[76 + 16 * i]))
                for i in range(k * 2)]
        zr = [(o, s) for o, s, m in ents if m == oracle.MODE_ZRUN]
        assert zr
        off, size = zr[0]
        cases = []
        b = blob.copy(); b[off] ^= 1; cases.append(("nnz", b))
        b = blob.copy(); b[off + 4] ^= 1; cases.append(("nblk", b))
        b = blob.copy(); b[off + 9] = 1; cases.append(("zeros", b))
        b = blob.copy(); b[off + 16] ^= 0x01; cases.append(("block bitmap", b))
        b = blob.copy(); b[off + size - 1] = 0; cases.append(("zero literal", b))
        nb = (65536 // 2 + 63) // 64
        l2 = 16 + ((nb + 7) // 8 + 15) // 16 * 16
        b = blob.copy(); b[off + l2] ^= 0x80; cases.append(("mask bit", b))
        ent = 64 + 16 * [i for i, (o, s, m) in enumerate(ents) if m == oracle.MODE_ZRUN][0]
        b = blob.copy(); b[ent + 12] = oracle.MODE_RAW; cases.append(("mode ZRUN -> RAW", b))
        for i in range(8):
            o, s = zr[int(rng.integers(0, len(zr)))]
            b = blob.copy()
            pos = o + int(rng.integers(0, s))
            b[pos] ^= 1 << int(rng.integers(0, 8))
            cases.append((f"zrun flip {pos}", b))
        for name, cb in cases:
            banner(f"delta corruption v2={shared} {name}")
            want_rc, want = oracle.decompress_delta(cb, x)
            hdr = bytes(cb[:64])
            d = torch.from_numpy(cb.copy()).cuda()
            info = ltc.blob_info(hdr)
            dst = torch.empty(info["nbytes"], dtype=torch.uint8, device="cuda")
            need = ltc.delta_workspace_size([hdr])
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
            status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
            ltc.decompress_delta_raw([hdr], [d.data_ptr()], [d.numel()], [tx.data_ptr()], [dst.data_ptr()],
                                     [dst.numel()], status.data_ptr(), ws.data_ptr(), ws.numel())
            st = int(status.item())
            assert st == want_rc, (name, st, want_rc)
            if st == 0:
                assert np.array_equal(dst.cpu().numpy(), want)
