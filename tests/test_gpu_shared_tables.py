"""GPU parity of blob format v2 (shared tables: one frequency table per stream
index, lmz README, "One format choice worth knowing about"): blobs written by
the HIP path must equal the oracle's v2 blobs byte for byte, v2 blobs must
decode to the input, and corrupted v2 blobs must get the oracle's verdict.
Inputs cover every dtype, ragged and one-element tensors, planes without a
table, random (RAW) chunks, batches split into chunk groups on several
streams, the checksums of compress_with_crc32 and the host-blob path.
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
    m.lib()
    return m


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def check_v2(ltc, arr, dtype, chunk=131072, thr=0.95, label=""):
    src = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
    banner(f"v2 case {label} dtype={dtype} chunk={chunk} thr={thr} bytes={src.size}")
    want = oracle.compress(src, dtype, chunk, thr, shared_tables=True)
    got = to_np_bytes(ltc.compress(to_gpu(src, dtype), chunk, thr, shared_tables=True))
    assert got.size == want.size, (got.size, want.size)
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError(f"v2 blob differs at {bad.size} bytes, first {bad[:8].tolist()}")
    out = ltc.decompress(torch.from_numpy(want.copy()).cuda())
    assert np.array_equal(to_np_bytes(out), src)
    return want


def test_c1(ltc):
    blob = check_v2(ltc, workloads.c1(), 1, label="C1")
    assert ltc.blob_info(bytes(blob[:64]))["version"] == 2


def test_fp32_and_fp16_slices(ltc):
    check_v2(ltc, workloads.c2().reshape(-1)[: 2 << 20], 3, label="C2 slice")
    clean, h = workloads.c4()
    check_v2(ltc, clean.reshape(-1)[: 1 << 20], 3, label="C4 clean slice (planes without tables)")
    check_v2(ltc, h.reshape(-1)[: 2 << 20], 2, label="C4 fp16 slice")


SMALL = [(d, n, c, k) for d in (0, 1, 2, 3) for n in (0, 1, 63, 1000, 5003, 70001)
         for c in (8, 24, 4096, 131072) for k in ("normal", "const", "random")
         if not (c == 8 and n > 5003)]


@pytest.mark.parametrize("dtype,nelem,chunk,kind", SMALL, ids=lambda v: str(v))
def test_small(ltc, dtype, nelem, chunk, kind):
    rng = np.random.default_rng(nelem * 7 + chunk + dtype)
    e = oracle.ELEM_BYTES[dtype]
    if kind == "normal":
        x = rng.standard_normal(nelem) * 0.02
        arr = {0: lambda: np.clip(np.rint(x * 2000) + 128, 0, 255).astype(np.uint8), 1: lambda: _bf16(x),
               2: lambda: x.astype(np.float16), 3: lambda: x.astype(np.float32)}[dtype]()
    elif kind == "const":
        arr = np.full(nelem * e, 0x3C, dtype=np.uint8)
    else:
        arr = rng.integers(0, 256, nelem * e, dtype=np.uint8)
    check_v2(ltc, arr, dtype, chunk, label=f"{kind} n={nelem}")


@pytest.mark.parametrize("thr", [1e-6, 0.5, 0.95, 1.0])
def test_thresholds(ltc, thr):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(300000) * np.repeat([0.02, 0.5, 1e-3], 100000)).astype(np.float32)
    check_v2(ltc, x, 3, 65536, thr, label="threshold")


@pytest.mark.parametrize("dtype,chunk", [(1, 8192), (3, 4096), (0, 2048)])
def test_grouped_with_random_chunks(ltc, dtype, chunk):
    """Over 4096 chunks: the tables come first, then two chunk groups.
    Chunks of a few thousand elements, so that streams are coded."""
    rng = np.random.default_rng(400 + dtype)
    nbytes = 4200 * chunk + 24
    if dtype == 0:
        data = rng.integers(0, 6, nbytes, dtype=np.uint8)
    else:
        x = (rng.standard_normal(nbytes // 4) * 0.02).astype(np.float32)
        data = (_bf16(x).view(np.uint8) if dtype == 1 else x.view(np.uint8))
        data = np.concatenate([data, data])[:nbytes]
    for c in range(0, nbytes // chunk, 5):
        data[c * chunk:(c + 1) * chunk] = rng.integers(0, 256, chunk, dtype=np.uint8)
    e = oracle.ELEM_BYTES[dtype]
    want = check_v2(ltc, data[: nbytes // e * e], dtype, chunk, label=f"grouped {dtype}")
    assert rans_streams(want) > 2000, rans_streams(want)


def test_batch_with_empty_and_tiny(ltc):
    rng = np.random.default_rng(79)
    chunk = 1024
    sizes = (90000, 0, 1, 123457, 2, 40000, 250001, 17, 60000)
    arrs = [(rng.standard_normal(n) * rng.choice([0.02, 1.0, 1e-4])).astype(np.float32) for n in sizes]
    ts = [to_gpu(a, 3) for a in arrs]
    blobs = ltc.compress_batch(ts, chunk, shared_tables=True)
    for a, b in zip(arrs, blobs):
        assert np.array_equal(to_np_bytes(b), oracle.compress(a, 3, chunk, shared_tables=True))
    outs = ltc.decompress_batch(blobs)
    for a, o in zip(arrs, outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))
    # v1 and v2 blobs decode side by side in one batch
    mixed = [blobs[0], ltc.compress(ts[3], chunk), blobs[6]]
    outs = ltc.decompress_batch(mixed)
    for a, o in zip((arrs[0], arrs[3], arrs[6]), outs):
        assert np.array_equal(to_np_bytes(o), a.view(np.uint8))


def test_checksums_and_host_path(ltc):
    x = workloads.c1()
    t = to_gpu(x, 1)
    blob, crc = ltc.compress_with_crc32(t, shared_tables=True)
    want = oracle.compress(x, 1, 131072, shared_tables=True)
    assert np.array_equal(to_np_bytes(blob), want)
    assert crc.cpu().numpy().view(np.uint32).tolist() == \
        [zlib.crc32(want[i:i + 16384].tobytes()) for i in range(0, want.size, 16384)]
    hb = ltc.compress_to_host(t, shared_tables=True)
    assert np.array_equal(hb.numpy(), want)
    assert torch.equal(ltc.decompress_from_host(hb).view(torch.int16), t.view(torch.int16))


def test_corrupt_v2_blobs_match_oracle_verdicts(ltc):
    rng = np.random.default_rng(11)
    x = _bf16(rng.standard_normal(200000) * 0.02)
    blob = oracle.compress(x, 1, 16384, shared_tables=True)
    k = int.from_bytes(blob[20:24].tobytes(), "little")
    t = 64 + 16 * k * 2
    base = int.from_bytes(blob[40:48].tobytes(), "little")
    cases = []
    b = blob.copy(); b[t + 16] ^= 1; cases.append(("plane 0 table sum", b))
    b = blob.copy(); b[base - 2] ^= 0x40; cases.append(("last table entry or pad", b))
    b = blob.copy(); b[t + 6] = 1; cases.append(("record zeros", b))
    b = blob.copy(); b[t + 2] = b[t]; b[t + 3] = b[t + 1]; cases.append(("lo == hi", b))
    b = blob.copy(); b[27] = 0; cases.append(("flags", b))
    b = blob.copy(); b[40] ^= 0x10; cases.append(("payload base", b))
    for i in range(8):
        b = blob.copy()
        pos = int(rng.integers(base, b.size))
        b[pos] ^= 1 << int(rng.integers(0, 8))
        cases.append((f"payload flip {pos}", b))
    for name, cb in cases:
        banner(f"v2 corruption {name}")
        want_rc, want = oracle.decompress(cb)
        hdr = bytes(cb[:64])
        try:
            info = ltc.blob_info(hdr)
        except ltc.LTCError as e:
            assert e.code == want_rc, (name, e.code, want_rc)
            continue
        d = torch.from_numpy(cb.copy()).cuda()
        dst = torch.empty(max(1, info["nbytes"]), dtype=torch.uint8, device="cuda")
        status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
        try:
            ltc.decompress_raw([hdr], [d.data_ptr()], [d.numel()], [dst.data_ptr()], [info["nbytes"]],
                               status.data_ptr())
        except ltc.LTCError as e:
            assert e.code == want_rc, (name, e.code, want_rc)
            continue
        st = int(status.item())
        assert st == want_rc, (name, st, want_rc)
        if st == 0:
            assert np.array_equal(dst[:info["nbytes"]].cpu().numpy(), want)
