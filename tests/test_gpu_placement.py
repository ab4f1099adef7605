"""GPU parity of top-last calls of 4096 chunks or more, where the encoder
writes the top streams' payloads into the blob itself: each wave publishes
its top streams' sizes and walks back over the statuses of the chunks before
them to find their offsets ("NOTE-241: ZipNN", Method item 5: the directory
maps every payload, so a payload's place follows from the sizes before it).

The cases make the walk meet everything it handles: chunks coded by the
128-entry and the 256-entry table launches in one tensor (the first launch
gives up behind a chunk left to the second, and k_pack writes those
payloads), top streams abandoned part way (their RAW fallback size enters
the sums), settled top streams (CONST, RAW by the size bound) published
before coding, tensors of one chunk and waves whose two chunks straddle two
tensors, format v2, every dtype, and the checksummed call.  Blobs must
equal the oracle's byte for byte.  Chunks hold
thousands of elements so that top streams are coded (a RANS payload carries
272 bytes of states and its table: a stream of 512 bytes never fits), and
each test checks in the oracle's directory that coded top streams are there.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import banner, stream_modes, to_gpu, to_np_bytes
from test_gpu_parity import _abandon_mix
from test_gpu_top_last import _bytes, _equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ltc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import lossless_tensor_compression_amd as m
    m.lib()
    return m


def _exp_chunks(dtype, kinds, chunk, rng):
    """One chunk per kind; the kind sets the top (exponent) byte: narrow
    (16 values), wide (two values far apart plus a few between: a 256-entry
    table), const (one value), uniform (RAW by the bound), a7 (90 values,
    about 6.5 bits: with 4096 elements the skip bound lets it be coded and the
    coder abandons it part way at threshold 0.88).  Sign and mantissa bytes
    are uniform."""
    e = oracle.ELEM_BYTES[dtype]
    n = chunk // e
    out = []
    for kind in kinds:
        if kind == "narrow":
            v = rng.integers(60, 76, n)
        elif kind == "wide":
            v = np.where(rng.random(n) < 0.5, 5, 240)
            v[rng.integers(0, n, 40)] = rng.integers(5, 241, 40)
        elif kind == "const":
            v = np.full(n, 99)
        elif kind == "uniform":
            v = rng.integers(0, 256, n)
        else:
            v = rng.integers(0, 90, n) + 40
        v = v.astype(np.uint64)
        if dtype == 0:
            out.append(v.astype(np.uint8))
        elif dtype == 1:
            low = rng.integers(0, 256, n).astype(np.uint64)
            out.append((((low >> 7) << 15) | (v << 7) | (low & 0x7F)).astype(np.uint16))
        else:
            m = rng.integers(0, 1 << 24, n).astype(np.uint64)
            out.append((((m >> 23) << 31) | (v << 23) | (m & 0x7FFFFF)).astype(np.uint32))
    return np.concatenate(out)


def _coded_tops(wants):
    return sum(int((stream_modes(w)[:, -1] == 1).sum()) for w in wants if len(w) > 64)


def _batch(ltc, arrs, dtype, chunk, thr=0.95, shared=False, crc=False, label="", min_coded=1000):
    chunks = sum((a.nbytes + chunk - 1) // chunk for a in arrs)
    assert chunks >= 4096, chunks  # the placed path
    banner(f"placement {label} dtype={dtype} chunk={chunk} chunks={chunks} thr={thr} v2={shared} crc={crc}")
    ts = [to_gpu(a, dtype) for a in arrs]
    if crc:
        blobs, crcs = ltc.compress_batch_with_crc32(ts, chunk, thr, 16384, shared_tables=shared, top_last=True)
    else:
        blobs = ltc.compress_batch(ts, chunk, thr, shared_tables=shared, top_last=True)
    wants = []
    for i, (a, b) in enumerate(zip(arrs, blobs)):
        want = oracle.compress(_bytes(a), dtype, chunk, thr, shared_tables=shared, top_last=True)
        _equal(to_np_bytes(b), want, f"{label} tensor {i}")
        if crc:
            got = crcs[i].cpu().numpy().view(np.uint32)
            assert np.array_equal(got, oracle.crc32_chunks(want, 16384)), i
        wants.append(want)
    assert _coded_tops(wants) >= min_coded, _coded_tops(wants)
    for a, o in zip(arrs, ltc.decompress_batch(blobs)):
        assert np.array_equal(to_np_bytes(o), _bytes(a))


@pytest.mark.parametrize("dtype", [0, 1, 3])
def test_both_table_launches_in_one_tensor(ltc, dtype):
    """Narrow, wide and mixed pairs along each tensor: in the 128-entry
    launch every wave behind a wide pair gives up and k_pack writes its
    payload; the 256-entry launch then places the wide ones."""
    rng = np.random.default_rng(500 + dtype)
    chunk = 8192 if dtype else 4096
    pattern = ["narrow"] * 40 + ["wide"] + ["narrow"] * 300 + ["wide", "wide"] + ["narrow"] * 37
    arrs = [_exp_chunks(dtype, pattern * 4, chunk, rng), _exp_chunks(dtype, pattern * 7, chunk, rng)]
    _batch(ltc, arrs, dtype, chunk, label="narrow and wide pairs")


@pytest.mark.parametrize("dtype", [1, 3])
def test_settled_abandoned_and_coded(ltc, dtype):
    """Every kind of top stream in the sums: coded, abandoned part way (RAW
    fallback size), CONST and RAW settled before coding."""
    rng = np.random.default_rng(520 + dtype)
    chunk = 8192 if dtype == 1 else 16384
    kinds = ["narrow", "a7", "const", "uniform", "narrow", "narrow", "a7", "a7", "narrow", "const"]
    x = _exp_chunks(dtype, kinds * 420, chunk, rng)
    _batch(ltc, [x], dtype, chunk, thr=0.88, label="abandoned at 0.88")
    _batch(ltc, [x], dtype, chunk, thr=0.95, label="all coded at 0.95", min_coded=2500)


def test_tensor_boundaries_and_tiny_tensors(ltc):
    """Tensors of one chunk, of an odd number of chunks (pairs straddling two
    tensors), empty and ragged tensors between long ones: every tensor's
    walk starts at its own first chunk."""
    rng = np.random.default_rng(540)
    chunk = 8192
    m = chunk // 2
    sizes = [1500 * m, 1, 0, m - 1, 1025 * m + 3, m, 3, 2001 * m + 77, 300, 2 * m]
    arrs = []
    for i, n in enumerate(sizes):
        a = (rng.standard_normal(n) * rng.choice([0.02, 1e-3, 0.3])).astype(np.float32)
        b = a.view(np.uint32) >> 16
        arrs.append(b.astype(np.uint16))
    _batch(ltc, arrs, 1, chunk, label="tensor boundaries")


@pytest.mark.parametrize("dtype", [1, 2])
def test_v2(ltc, dtype):
    """Format v2: the plane tables, the RAW streams named by k_decide and
    written by the encoder, the 128-entry launch for narrow streams."""
    rng = np.random.default_rng(560 + dtype)
    chunk = 8192
    n = 4100 * chunk // 2
    a = (rng.standard_normal(n) * 0.02).astype(np.float32)
    x = (a.view(np.uint32) >> 16).astype(np.uint16) if dtype == 1 else a.astype(np.float16).view(np.uint16)
    _batch(ltc, [x[: n // 2], x[n // 2:]], dtype, chunk, shared=True, label="v2")


def test_checksummed_call(ltc):
    rng = np.random.default_rng(580)
    chunk = 8192
    kinds = ["narrow", "wide", "narrow", "uniform", "narrow", "narrow", "const", "narrow"]
    x = _exp_chunks(1, kinds * 520, chunk, rng)
    cut = 1000 * chunk // 2 + 5
    _batch(ltc, [x[:cut], x[cut:]], 1, chunk, crc=True, label="compress_with_crc32")


def test_abandon_mix_full_chunks(ltc):
    """The exponent mixes of the staged-stream tests, at the default chunk
    size over 4096 chunks (512 MiB of BF16)."""
    rng = np.random.default_rng(600)
    bits = [7, 5, 5, 7, 7, 5, 7, 5, 5] * 456
    x = _abandon_mix(1, bits, 131072, rng)
    _batch(ltc, [x], 1, 131072, thr=0.88, label="512 MiB abandon mix")


def test_two_streams_per_wave(ltc):
    """16,384 chunks or more: the encoder codes two chunks' streams per wave
    and places both payloads (the second takes the first's prefix when both
    are in one tensor); narrow, wide, abandoned, constant and RAW top
    streams, and tensors that end on odd chunks."""
    rng = np.random.default_rng(620)
    chunk = 8192
    m = chunk // 2
    kinds = ["narrow", "narrow", "wide", "a7", "narrow", "const", "uniform", "narrow", "narrow", "a7", "narrow"]
    x = _exp_chunks(1, kinds * 1500, chunk, rng)  # 16,500 chunks
    cut = [0, 4001 * m, 4002 * m, 11001 * m, x.size]
    _batch(ltc, [x[a:b] for a, b in zip(cut, cut[1:])], 1, chunk, thr=0.88, label="two streams per wave",
           min_coded=8000)


def _raw_call(ltc, arrs, dtype, chunk, flags, thr, crc):
    ts = [to_gpu(a, dtype) for a in arrs]
    nbytes = [a.nbytes for a in arrs]
    caps = [ltc.compress_bound(n, dtype, chunk) for n in nbytes]
    ws_n = ltc.workspace_size(nbytes, dtype, chunk)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    blobs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    sizes = torch.zeros(len(ts), dtype=torch.int64, device="cuda")
    ccap = [(c + crc - 1) // crc for c in caps] if crc else None
    crcs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in ccap] if crc else None
    ltc.compress_ex_raw([t.data_ptr() for t in ts], nbytes, dtype, chunk, thr, flags,
                        [b.data_ptr() for b in blobs], caps, sizes.data_ptr(), ws.data_ptr(), ws_n,
                        crc, [c.data_ptr() for c in crcs] if crc else None, ccap)
    torch.cuda.synchronize()
    out = []
    for i, (b, s) in enumerate(zip(blobs, sizes.cpu().tolist())):
        got = crcs[i][:(s + crc - 1) // crc].cpu().numpy().view(np.uint32) if crc else None
        out.append((to_np_bytes(b[:s]), got))
    return out


@pytest.mark.parametrize("case", ["both launches", "two streams per wave"])
@pytest.mark.parametrize("crc", [0, 16384])
def test_no_wait_leaves_payloads_to_packing(ltc, case, crc):
    """LTC_FLAG_PLACE_NO_WAIT: a placing wave gives up at the first size it
    does not find (the fallback a predecessor slower than the wait bound
    triggers), so the payloads behind any chunk still coding go to k_pack
    instead.  Blobs and checksums must still equal the oracle's: the walk
    only decides who writes a payload, never where."""
    rng = np.random.default_rng(640 + len(case) + crc)
    chunk = 8192
    m = chunk // 2
    if case == "both launches":
        pattern = ["narrow"] * 40 + ["wide"] + ["narrow"] * 300 + ["wide", "wide"] + ["narrow"] * 37
        arrs = [_exp_chunks(1, pattern * 5, chunk, rng), _exp_chunks(1, pattern * 7, chunk, rng)]
        thr = 0.95
    else:
        kinds = ["narrow", "narrow", "wide", "a7", "narrow", "const", "uniform", "narrow", "narrow", "a7", "narrow"]
        x = _exp_chunks(1, kinds * 1500, chunk, rng)
        cut = [0, 5003 * m, 5004 * m, 12001 * m, x.size]
        arrs = [x[a:b] for a, b in zip(cut, cut[1:])]
        thr = 0.88
    assert sum((a.nbytes + chunk - 1) // chunk for a in arrs) >= 4096  # the placed path
    banner(f"no-wait placement {case} crc={crc}")
    got = _raw_call(ltc, arrs, 1, chunk, ltc.FLAG_TOP_LAST | ltc.FLAG_PLACE_NO_WAIT, thr, crc)
    wants = []
    for i, (a, (blob, c)) in enumerate(zip(arrs, got)):
        want = oracle.compress(_bytes(a), 1, chunk, thr, top_last=True)
        _equal(blob, want, f"{case} tensor {i}")
        if crc:
            assert np.array_equal(c, oracle.crc32_chunks(want, crc)), i
        wants.append(want)
    assert _coded_tops(wants) >= 2000, _coded_tops(wants)
