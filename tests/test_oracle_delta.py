"""Pins for the oracle's deltas ("NOTE-241: ZipNN", Method item 6 and the
Deltas results: XOR against a base, then a run coder instead of the order-0
coder when more than 90% of a byte group is zero bytes or a zero run exceeds
3% of it).

What fixes them independently of the oracle's delta code:
- with no ZRUN stream, a delta blob is the plain blob of src XOR base (numpy)
  with the delta flag set, byte for byte;
- every ZRUN payload, parsed with numpy, rebuilds the chunk stream of
  src XOR base gathered with numpy, and has the size the layout gives;
- the coder choice follows the rule and the sizes: the rule from numpy's
  zero count and longest zero run, the RANS size from the plain rANS encoder
  with the v1 table of the stream;
- identical tensors give only CONST streams; decoding needs the base.
"""
import struct

import numpy as np
import pytest
import torch

import oracle
import workloads


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def _reorder_np(dtype, x):
    if dtype == 0:
        return x.astype(np.uint32)
    w, wm = {1: (16, 7), 2: (16, 10), 3: (32, 23)}[dtype]
    x = x.astype(np.uint64)
    e = (x >> wm) & ((1 << (w - 1 - wm)) - 1)
    s = (x >> (w - 1)) & 1
    m = x & ((1 << wm) - 1)
    return ((e << (wm + 1)) | (s << wm) | m).astype(np.uint32)


def _streams(src_bytes, dtype, chunk):
    e = oracle.ELEM_BYTES[dtype]
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[e]
    out = []
    for c0 in range(0, src_bytes.size, chunk):
        y = _reorder_np(dtype, src_bytes[c0:c0 + chunk].view(dt))
        out.append([((y >> (8 * k)) & 0xFF).astype(np.uint8) for k in range(e)])
    return out


def _zrun_parse(pl, n):
    nnz, nblk = struct.unpack_from("<II", pl, 0)
    assert not pl[8:16].any()
    nb = (n + 63) // 64
    l1 = np.unpackbits(pl[16:16 + (nb + 7) // 8], bitorder="little")[:nb]
    l2 = 16 + ((nb + 7) // 8 + 15) // 16 * 16
    lit = l2 + (8 * nblk + 15) // 16 * 16
    assert pl.size == lit + nnz and int(l1.sum()) == nblk
    masks = np.frombuffer(pl[l2:l2 + 8 * nblk].tobytes(), dtype="<u8")
    out = np.zeros(nb * 64, dtype=np.uint8)
    blocks = np.nonzero(l1)[0]
    bits = np.unpackbits(masks.view(np.uint8), bitorder="little").reshape(-1, 64).astype(bool)
    pos = (blocks[:, None] * 64 + np.arange(64)[None, :])[bits]
    assert pos.size == nnz
    out[pos] = pl[lit:lit + nnz]
    assert (out[pos] != 0).all() and not out[n:].any()
    return out[:n]


def _rule(sym):
    n = sym.size
    zeros = int((sym == 0).sum())
    z = np.concatenate([[0], (sym == 0).astype(np.int64), [0]])
    d = np.diff(z)
    starts, ends = np.nonzero(d == 1)[0], np.nonzero(d == -1)[0]
    longest = int((ends - starts).max()) if starts.size else 0
    return 10 * zeros > 9 * n or 100 * longest > 3 * n


def _cases():
    rng = np.random.default_rng(21)
    x = workloads.c1()[:300_000]
    # fine-tuning-like: 10% of the elements nudged by a few ulps
    y = x.copy()
    idx = rng.choice(y.size, y.size // 10, replace=False)
    y[idx] = (y[idx].astype(np.int32) + rng.integers(-3, 4, idx.size)).astype(y.dtype)
    yield "bf16 sparse nudges", 1, 65536, y, x
    # long unchanged runs then a dense change: the run coder's case
    z = x.copy()
    for c0 in range(0, z.size, 32768):
        z[c0 + 24000:c0 + 32768] = rng.integers(0, 65536, z[c0 + 24000:c0 + 32768].size).astype(z.dtype)
    yield "bf16 unchanged runs", 1, 65536, z, x
    f = (rng.standard_normal(70_001) * 0.02).astype(np.float32)
    g = f.copy()
    g[::7] += np.float32(1e-6)
    yield "fp32 every 7th", 3, 65536, g, f
    u = rng.integers(0, 4, 50_000, dtype=np.uint8)
    v = u.copy()
    v[10_000:11_000] ^= rng.integers(1, 256, 1_000, dtype=np.uint8)
    yield "u8 one burst", 0, 4096, v, u


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: c[0])
def test_delta_against_numpy(case):
    name, dtype, chunk, src, base = case
    sb = np.ascontiguousarray(src).reshape(-1).view(np.uint8)
    bb = np.ascontiguousarray(base).reshape(-1).view(np.uint8)
    xor = sb ^ bb
    blob = oracle.compress_delta(sb, bb, dtype, chunk)
    assert blob[27] == oracle.FLAG_DELTA and struct.unpack_from("<H", blob, 4)[0] == 1
    e = oracle.ELEM_BYTES[dtype]
    k = struct.unpack_from("<I", blob, 20)[0]
    ents = [struct.unpack_from("<QIBBH", blob, 64 + 16 * i) for i in range(k * e)]
    modes = np.array([m for _, _, m, _, _ in ents])
    streams = _streams(xor, dtype, chunk)
    for i, (off, size, mode, cval, _) in enumerate(ents):
        c, q = divmod(i, e)
        sym = streams[c][q]
        if mode == oracle.MODE_CONST:
            assert (sym == cval).all()
            continue
        if mode == oracle.MODE_ZRUN:
            assert np.array_equal(_zrun_parse(blob[off:off + size], sym.size), sym)
        h = oracle.histogram(sym)
        assert np.count_nonzero(h) >= 2
        f = oracle.normalize(h)
        _, words = oracle.rans_encode(sym, f)
        lo, hi = np.nonzero(h)[0][[0, -1]]
        p_rans = (272 + 2 * (hi - lo + 1) + 15) // 16 * 16 + 2 * words.size
        nb = (sym.size + 63) // 64
        nzb = int(np.count_nonzero(np.pad(sym, (0, nb * 64 - sym.size)).reshape(nb, 64).any(axis=1)))
        p_z = 16 + ((nb + 7) // 8 + 15) // 16 * 16 + (8 * nzb + 15) // 16 * 16 + int((sym != 0).sum())
        pmax = oracle.p_max(sym.size, 0.95)
        use_z = _rule(sym) and p_z < p_rans and p_z <= pmax
        if use_z:
            assert (mode, size) == (oracle.MODE_ZRUN, p_z), (name, i)
        elif p_rans <= pmax:
            assert (mode, size) == (oracle.MODE_RANS, p_rans), (name, i)
        else:
            assert (mode, size) == (oracle.MODE_RAW, sym.size), (name, i)
    if not (modes == oracle.MODE_ZRUN).any():
        plain = oracle.compress(xor, dtype, chunk)
        plain[27] = oracle.FLAG_DELTA
        assert np.array_equal(blob, plain)
    rc, out = oracle.decompress_delta(blob, bb)
    assert rc == 0 and np.array_equal(out, sb)
    # a v2 delta blob decodes to the same bytes
    b2 = oracle.compress_delta(sb, bb, dtype, chunk, shared_tables=True)
    assert b2[27] == oracle.FLAG_DELTA | oracle.FLAG_SHARED_TABLES
    rc, out = oracle.decompress_delta(b2, bb)
    assert rc == 0 and np.array_equal(out, sb)


def test_both_coders_occur():
    """The cases above exercise ZRUN and RANS streams in delta blobs."""
    seen = set()
    for name, dtype, chunk, src, base in _cases():
        sb = np.ascontiguousarray(src).reshape(-1).view(np.uint8)
        bb = np.ascontiguousarray(base).reshape(-1).view(np.uint8)
        blob = oracle.compress_delta(sb, bb, dtype, chunk)
        k = struct.unpack_from("<I", blob, 20)[0]
        e = oracle.ELEM_BYTES[dtype]
        seen |= set(blob[64 + 12:64 + 16 * k * e:16].tolist())
    assert oracle.MODE_ZRUN in seen and oracle.MODE_RANS in seen


def test_identical_tensors_and_base_rules():
    x = workloads.c1()[:100_000]
    blob = oracle.compress_delta(x, x, 1, 16384)
    k = struct.unpack_from("<I", blob, 20)[0]
    assert (blob[64 + 12:64 + 16 * k * 2:16] == oracle.MODE_CONST).all()
    assert (blob[64 + 13:64 + 16 * k * 2:16] == 0).all()
    assert blob.size == 64 + 16 * k * 2
    # a delta blob needs its base, a plain blob takes none
    assert oracle.decompress(blob)[0] == oracle.ERR_INVALID_ARGUMENT
    assert oracle.decompress_delta(oracle.compress(x, 1), x)[0] == oracle.ERR_INVALID_ARGUMENT
    rc, out = oracle.decompress_delta(blob, x)
    assert rc == 0 and np.array_equal(out, x.view(np.uint8))


def test_tiny_u8_brute_force():
    """Every U8 pair (src, base) of length 0..3 over {0, 1, 200}, chunk 8."""
    import itertools
    vals = [0, 1, 200]
    for n in range(4):
        for s in itertools.product(vals, repeat=n):
            for b in itertools.product(vals, repeat=n):
                src = np.array(s, dtype=np.uint8)
                base = np.array(b, dtype=np.uint8)
                blob = oracle.compress_delta(src, base, 0, 8)
                rc, out = oracle.decompress_delta(blob, base)
                assert rc == 0 and out.tobytes() == src.tobytes()


def test_corrupt_zrun_payloads():
    rng = np.random.default_rng(4)
    x = workloads.c1()[:200_000]
    z = x.copy()
    for c0 in range(0, z.size, 32768):
        z[c0 + 24000:c0 + 32768] = rng.integers(0, 65536, z[c0 + 24000:c0 + 32768].size).astype(z.dtype)
    blob = oracle.compress_delta(z, x, 1, 65536)
    k = struct.unpack_from("<I", blob, 20)[0]
    ents = [struct.unpack_from("<QIBBH", blob, 64 + 16 * i) for i in range(k * 2)]
    zr = [(o, s) for o, s, m, _, _ in ents if m == oracle.MODE_ZRUN]
    assert zr
    off, size = zr[0]
    cases = []
    b = blob.copy(); b[off] ^= 1; cases.append(("nnz", b))
    b = blob.copy(); b[off + 4] ^= 1; cases.append(("nblk", b))
    b = blob.copy(); b[off + 9] = 1; cases.append(("zeros", b))
    b = blob.copy(); b[off + 16] ^= 0x01; cases.append(("block bitmap", b))
    b = blob.copy(); b[off + size - 1] = 0; cases.append(("zero literal", b))
    for name, cb in cases:
        rc, _ = oracle.decompress_delta(cb, x)
        assert rc == oracle.ERR_CORRUPT, name
