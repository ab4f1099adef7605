"""Pins for the oracle's top-last layout (header flag 8): the payload of stream
E-1 of every chunk placed after all other payloads.  NOTE-241: ZipNN,
"Method" item 5: the map of variable-size compressed pieces (the directory)
says where each one is, so the order of the payloads is a layout choice.

What fixes it independently of the oracle's placement code:
- hand-assembled blobs (tests/golden/top_last.json) for BF16 and FP32; the
  FP32 one tells the layout apart from both directory order and a
  plane-by-plane order;
- against the blob without the flag (itself pinned by tests/golden/blobs.json
  and the brute-force tests): same size, header but for the flag byte, same
  directory but for the offsets, the same payload bytes behind every entry,
  and offsets that follow the top-last order (walked here with numpy);
- the decoder's verdicts: a blob's offsets must follow the order its flag
  names.
"""
import json
import os
import struct

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "top_last.json")))["cases"]


def _hex(s):
    return bytes.fromhex(s.replace(" ", ""))


@pytest.mark.parametrize("case", GOLDEN, ids=lambda c: c["name"])
def test_golden_top_last(case):
    src = np.frombuffer(_hex(case["input_hex"]), dtype=np.uint8).copy()
    blob = oracle.compress(src, case["dtype"], case["chunk_bytes"], case["threshold"], top_last=True)
    assert blob.tobytes() == _hex(case["hex"]), case["derivation"]
    rc, out = oracle.decompress(blob)
    assert rc == 0 and out.tobytes() == src.tobytes()


def _entries(blob):
    k, e = struct.unpack_from("<I", blob, 20)[0], int(blob[7])
    out = []
    for i in range(k * e):
        off, size, mode, cval, z = struct.unpack_from("<QIBBH", blob, 64 + 16 * i)
        out.append((off, size, mode, cval, z))
    return k, e, out


def _top_last_order(k, e):
    lower = [c * e + q for c in range(k) for q in range(e - 1)]
    return lower + [c * e + e - 1 for c in range(k)]


def _inputs():
    rng = np.random.default_rng(11)
    x = workloads.c1()
    f32 = (rng.standard_normal(9001) * 0.03).astype(np.float32)
    clean = f32.view(np.uint32) & np.uint32(0xFFFF0000)  # low bytes CONST
    f16 = (rng.standard_normal(20000) * 0.1).astype(np.float16)
    u8 = rng.integers(0, 9, 7777).astype(np.uint8)
    return [
        ("bf16-c1", x, 1, 131072),
        ("bf16-c1-ragged", x[:123457], 1, 16384),
        ("fp32-ragged", f32, 3, 4096),
        ("fp32-clean", clean.view(np.float32), 3, 8192),
        ("fp16", f16, 2, 8192),
        ("u8", u8, 0, 1024),
        ("empty", np.zeros(0, np.uint8), 1, 4096),
        ("one-element", x[:1], 1, 4096),
    ]


@pytest.mark.parametrize("shared", [False, True], ids=["v1", "v2"])
@pytest.mark.parametrize("name,x,dtype,chunk", _inputs(), ids=[i[0] for i in _inputs()])
def test_same_payloads_as_directory_order(name, x, dtype, chunk, shared):
    a = oracle.compress(x, dtype, chunk, shared_tables=shared)
    b = oracle.compress(x, dtype, chunk, shared_tables=shared, top_last=True)
    check_relation(a, b)
    rc, out = oracle.decompress(b)
    assert rc == 0 and out.tobytes() == np.ascontiguousarray(x).tobytes()


def check_relation(a, b):
    """b: the top-last blob of the same input as the untagged blob a."""
    assert a.size == b.size
    assert int(b[27]) == int(a[27]) | 8
    assert a[:27].tobytes() == b[:27].tobytes() and a[28:64].tobytes() == b[28:64].tobytes()
    k, e, ea = _entries(a)
    _, _, eb = _entries(b)
    base = struct.unpack_from("<Q", a, 40)[0]
    # tables (v2) between the directory and payload_base are unchanged
    assert a[64 + 16 * k * e:base].tobytes() == b[64 + 16 * k * e:base].tobytes()
    cur = base
    for i in _top_last_order(k, e):
        off, size, mode, cval, z = eb[i]
        assert (size, mode, cval, z) == ea[i][1:]
        assert off == cur
        assert b[off:off + size].tobytes() == a[ea[i][0]:ea[i][0] + size].tobytes()
        cur = (off + size + 15) // 16 * 16
    assert cur == b.size
    # every gap byte is zero
    used = np.zeros(b.size, bool)
    used[:base] = True
    for off, size, *_ in eb:
        used[off:off + size] = True
    assert not b[~used].any()


def test_deltas():
    rng = np.random.default_rng(5)
    base = workloads.c1()[:200000]
    src = base.copy()
    src[rng.integers(0, src.size, 3000)] ^= 1
    for shared in (False, True):
        a = oracle.compress_delta(src, base, 1, 16384, shared_tables=shared)
        b = oracle.compress_delta(src, base, 1, 16384, shared_tables=shared, top_last=True)
        check_relation(a, b)
        rc, out = oracle.decompress_delta(b, base)
        assert rc == 0 and out.tobytes() == src.tobytes()


def test_u8_orders_coincide():
    u8 = np.random.default_rng(2).integers(0, 5, 5000).astype(np.uint8)
    a = oracle.compress(u8, 0, 512)
    b = oracle.compress(u8, 0, 512, top_last=True)
    assert b[27] == 8 and a[27] == 0
    a[27] = 8
    assert a.tobytes() == b.tobytes()


def test_order_must_match_the_flag():
    x = workloads.c1()[:300000]
    a = oracle.compress(x, 1, 16384)
    b = oracle.compress(x, 1, 16384, top_last=True)
    assert a.tobytes() != b.tobytes()
    for blob, flip in ((a, 8), (b, 8)):
        c = blob.copy()
        c[27] ^= flip  # claims the other order
        assert oracle.decompress(c)[0] == -5
    c = b.copy()
    c[27] |= 16  # an unknown flag bit
    assert oracle.decompress(c)[0] == -5
    # two top payloads swapped in place (entries still self-consistent in size)
    k, e, eb = _entries(b)
    i, j = 1, 3  # top streams of chunks 0 and 1
    c = b.copy()
    oi, oj = eb[i][0], eb[j][0]
    struct.pack_into("<Q", c, 64 + 16 * i, oj)
    struct.pack_into("<Q", c, 64 + 16 * j, oi)
    assert oracle.decompress(c)[0] == -5


def test_rejects_unknown_compress_flags():
    x = workloads.c1()[:1000]
    lib = oracle.lib()
    import ctypes
    blob = np.zeros(100000, np.uint8)
    nb = ctypes.c_uint64(0)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
    xb = x.view(np.uint8)
    assert lib.ltco_compress_ex(p(xb), xb.size, 1, 4096, 0.95, 4, p(blob), blob.size, ctypes.byref(nb), 1) == -1
    assert lib.ltco_compress_ex(p(xb), xb.size, 1, 4096, 0.95, 9, p(blob), blob.size, ctypes.byref(nb), 1) == 0
