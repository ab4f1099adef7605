"""Pins for the oracle's format v2 (shared tables: one frequency table per
stream index, lmz README, "One format choice worth knowing about").

What fixes v2 independently of the oracle's own v2 code:
- the table record of plane k is the v1 normalisation of the histogram of
  all of the blob's stream-k bytes, which the tests gather with numpy;
- every RANS payload decodes, with the plain rANS decoder and that table,
  to the chunk's stream bytes gathered with numpy;
- a one-chunk tensor's plane table is the chunk's own table, so its v2 payload
  carries exactly the states and words of the v1 payload;
- header, record and offset layout written out field by field;
- round trips over awkward shapes, and corrupted tables rejected.
"""
import struct

import numpy as np
import pytest
import torch

import oracle


def _reorder_np(dtype, x):
    """Exponent to the top byte, sign below it, mantissa in place."""
    if dtype == 0:
        return x.astype(np.uint32)
    w, wm = {1: (16, 7), 2: (16, 10), 3: (32, 23)}[dtype]
    x = x.astype(np.uint64)
    e = (x >> wm) & ((1 << (w - 1 - wm)) - 1)
    s = (x >> (w - 1)) & 1
    m = x & ((1 << wm) - 1)
    return ((e << (wm + 1)) | (s << wm) | m).astype(np.uint32)


def _streams(src_bytes, dtype, chunk):
    """streams[c][k] = byte k of every reordered element of chunk c."""
    e = oracle.ELEM_BYTES[dtype]
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[e]
    out = []
    for c0 in range(0, src_bytes.size, chunk):
        el = src_bytes[c0:c0 + chunk].view(dt)
        y = _reorder_np(dtype, el)
        out.append([((y >> (8 * k)) & 0xFF).astype(np.uint8) for k in range(e)])
    return out


def _parse_v2(blob):
    assert blob[:4].tobytes() == b"LTCB"
    ver, dtype, e = struct.unpack_from("<HBB", blob, 4)
    n, chunk, k = struct.unpack_from("<QII", blob, 8)
    lanes, pbits, flags, z = struct.unpack_from("<HBBI", blob, 24)
    bn, base = struct.unpack_from("<QQ", blob, 32)
    assert (ver, lanes, pbits, flags, z) == (2, 64, 12, 1, 0) and bn == blob.size
    assert not blob[48:64].any()
    s = k * e
    ents = [struct.unpack_from("<QIBBH", blob, 64 + 16 * i) for i in range(s)]
    t = 64 + 16 * s
    tables = []
    for q in range(e):
        lo, hi = struct.unpack_from("<HH", blob, t)
        assert not blob[t + 4:t + 16].any()
        if (lo, hi) == (1, 0):
            tables.append(None)
            t += 16
            continue
        f = np.zeros(256, dtype=np.uint16)
        f[lo:hi + 1] = np.frombuffer(blob[t + 16:t + 16 + 2 * (hi - lo + 1)].tobytes(), dtype="<u2")
        rb = (16 + 2 * (hi - lo + 1) + 15) // 16 * 16
        assert not blob[t + 16 + 2 * (hi - lo + 1):t + rb].any()
        tables.append(f)
        t += rb
    assert base == t
    return dict(dtype=dtype, e=e, n=n, chunk=chunk, k=k, ents=ents, tables=tables, base=base)


def _payload(blob, off, size):
    w = struct.unpack_from("<I", blob, off)[0]
    assert not blob[off + 4:off + 16].any() and size == 272 + 2 * w
    states = np.frombuffer(blob[off + 16:off + 272].tobytes(), dtype="<u4").copy()
    words = np.frombuffer(blob[off + 272:off + 272 + 2 * w].tobytes(), dtype="<u2").copy()
    return states, words


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


CASES = [
    ("bf16 mixed sigma", 1, 16384, lambda r: _bf16(r.standard_normal(50_000) * np.repeat([0.02, 0.5], 25_000))),
    ("fp32 normal", 3, 65536, lambda r: (r.standard_normal(70_001) * 0.02).astype(np.float32)),
    ("fp16 normal", 2, 4096, lambda r: (r.standard_normal(20_000) * 0.1).astype(np.float16)),
    ("u8 skewed", 0, 1000, lambda r: r.integers(0, 6, 9_999, dtype=np.uint8)),
    ("bf16 one chunk", 1, 131072, lambda r: _bf16(r.standard_normal(40_000) * 0.02)),
    ("fp32 const low bytes", 3, 8192, lambda r: (_bf16(r.standard_normal(10_000) * 0.02).astype(np.uint32) << 16).view(np.float32)),
]


@pytest.mark.parametrize("name,dtype,chunk,gen", CASES, ids=[c[0] for c in CASES])
def test_tables_and_payloads_against_numpy(name, dtype, chunk, gen):
    src = np.ascontiguousarray(gen(np.random.default_rng(len(name)))).reshape(-1).view(np.uint8)
    blob = oracle.compress(src, dtype, chunk, 0.95, shared_tables=True)
    p = _parse_v2(blob)
    streams = _streams(src, dtype, chunk)
    e = p["e"]
    assert p["k"] == len(streams)
    for q in range(e):
        plane = np.concatenate([st[q] for st in streams]) if streams else np.zeros(0, np.uint8)
        h = np.bincount(plane, minlength=256).astype(np.uint64)
        if np.count_nonzero(h) < 2:
            assert p["tables"][q] is None
        else:
            assert np.array_equal(p["tables"][q], oracle.normalize(h)), (name, q)
    cursor = p["base"]
    for i, (off, size, mode, cval, z) in enumerate(p["ents"]):
        c, q = divmod(i, e)
        sym = streams[c][q]
        assert off == cursor and z == 0
        cursor = (off + size + 15) // 16 * 16
        if np.count_nonzero(np.bincount(sym, minlength=256)) == 1:
            assert (mode, size, cval) == (oracle.MODE_CONST, 0, int(sym[0]))
            continue
        states, words = oracle.rans_encode(sym, p["tables"][q])
        coded = 272 + 2 * words.size
        if coded <= oracle.p_max(sym.size, 0.95):
            assert (mode, size) == (oracle.MODE_RANS, coded)
            st, wd = _payload(blob, off, size)
            assert np.array_equal(st, states) and np.array_equal(wd, words)
            rc, dec = oracle.rans_decode(wd, st, p["tables"][q], sym.size)
            assert rc == 0 and np.array_equal(dec, sym)
        else:
            assert (mode, size) == (oracle.MODE_RAW, sym.size)
            assert np.array_equal(blob[off:off + size], sym)
    assert cursor == blob.size
    rc, out = oracle.decompress(blob)
    assert rc == 0 and np.array_equal(out, src)


def test_one_chunk_tensor_carries_the_v1_states_and_words():
    rng = np.random.default_rng(3)
    for dtype, arr in ((1, _bf16(rng.standard_normal(30_000) * 0.02)),
                       (3, (rng.standard_normal(8_000) * 0.02).astype(np.float32))):
        src = arr.view(np.uint8)
        v1 = oracle.compress(src, dtype, 131072)
        v2 = oracle.compress(src, dtype, 131072, shared_tables=True)
        p = _parse_v2(v2)
        e = p["e"]
        for q in range(e):
            o1, s1, m1, _, _ = struct.unpack_from("<QIBBH", v1, 64 + 16 * q)
            o2, s2, m2, _, _ = p["ents"][q]
            assert m1 == m2
            if m1 != oracle.MODE_RANS:
                continue
            w1 = struct.unpack_from("<I", v1, o1)[0]
            lo, hi = int(v1[o1 + 4]), int(v1[o1 + 5])
            f1 = np.frombuffer(v1[o1 + 272:o1 + 272 + 2 * (hi - lo + 1)].tobytes(), dtype="<u2")
            assert np.array_equal(p["tables"][q][lo:hi + 1], f1)
            assert p["tables"][q][:lo].sum() == 0 and p["tables"][q][hi + 1:].sum() == 0
            wo = (272 + 2 * (hi - lo + 1) + 15) // 16 * 16
            st, wd = _payload(v2, o2, s2)
            assert np.array_equal(st, np.frombuffer(v1[o1 + 16:o1 + 272].tobytes(), dtype="<u4"))
            assert np.array_equal(wd, np.frombuffer(v1[o1 + wo:o1 + wo + 2 * w1].tobytes(), dtype="<u2"))


@pytest.mark.parametrize("dtype", [0, 1, 2, 3])
@pytest.mark.parametrize("nelem,chunk", [(0, 8), (1, 8), (7, 8), (1000, 24), (5003, 4096), (70001, 131072)])
def test_round_trip_awkward(dtype, nelem, chunk):
    rng = np.random.default_rng(nelem + dtype)
    e = oracle.ELEM_BYTES[dtype]
    for kind in ("normal", "const", "random"):
        if kind == "normal":
            x = rng.standard_normal(nelem) * 0.02
            arr = {0: lambda: np.clip(np.rint(x * 2000) + 128, 0, 255).astype(np.uint8), 1: lambda: _bf16(x),
                   2: lambda: x.astype(np.float16), 3: lambda: x.astype(np.float32)}[dtype]()
        elif kind == "const":
            arr = np.full(nelem * e, 0x3C, dtype=np.uint8)
        else:
            arr = rng.integers(0, 256, nelem * e, dtype=np.uint8)
        src = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
        blob = oracle.compress(src, dtype, chunk, shared_tables=True)
        assert blob.size <= oracle.compress_bound(src.size, dtype, chunk, shared_tables=True)
        _parse_v2(blob)
        rc, out = oracle.decompress(blob)
        assert rc == 0 and np.array_equal(out, src), (kind, dtype, nelem, chunk)


def test_corrupt_tables_and_versions():
    rng = np.random.default_rng(9)
    src = _bf16(rng.standard_normal(40_000) * 0.02).view(np.uint8)
    blob = oracle.compress(src, 1, 16384, shared_tables=True)
    p = _parse_v2(blob)
    t = 64 + 16 * p["k"] * p["e"]
    q = next(i for i, tb in enumerate(p["tables"]) if tb is not None)
    for i in range(q):
        t += 16 if p["tables"][i] is None else 0
    lo = struct.unpack_from("<H", blob, t)[0]
    cases = []
    b = blob.copy(); b[t + 16] ^= 1; cases.append(("table sum", b))          # f[lo] changes
    b = blob.copy(); b[t + 2] = b[t]; b[t + 3] = b[t + 1]; cases.append(("lo == hi", b))
    b = blob.copy(); b[t + 5] = 1; cases.append(("record zeros", b))
    b = blob.copy(); b[4] = 3; cases.append(("version 3", b))
    b = blob.copy(); b[27] = 0; cases.append(("flags", b))
    for name, cb in cases:
        rc, _ = oracle.decompress(cb)
        assert rc in (oracle.ERR_CORRUPT, oracle.ERR_BAD_VERSION), (name, rc)
    assert oracle.decompress(cases[3][1])[0] == oracle.ERR_BAD_VERSION
    assert lo < 256
