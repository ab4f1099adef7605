"""CPU oracle for the lossless tensor codec (ctypes over libltc_oracle.so).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  It is a plain, slow,
scalar C implementation of the blob format described in ltc_oracle.h, written
independently of the HIP library; the two share no code.

The functions here only marshal numpy arrays to the C entry points.
"""
import ctypes
import os

import numpy as np

from . import build as _build

DTYPES = {"u8": 0, "bf16": 1, "fp16": 2, "fp32": 3}
ELEM_BYTES = {0: 1, 1: 2, 2: 2, 3: 4}
MODE_RAW, MODE_RANS, MODE_CONST, MODE_ZRUN = 0, 1, 2, 3
FLAG_SHARED_TABLES = 1  # format v2: one frequency table per stream index
FLAG_DELTA = 2          # header flag: XOR delta against a base
FLAG_TOP_LAST = 8       # layout: top-stream payloads after all others

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED_DTYPE = -2
ERR_BAD_MAGIC = -3
ERR_BAD_VERSION = -4
ERR_CORRUPT = -5
ERR_CAPACITY = -6

_lib = None


def _u8p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def lib():
    global _lib
    if _lib is None:
        # LTC_ORACLE_LIB: another build of the same source (the sanitized one
        # of tests/test_host_sanitized.py)
        path = os.environ.get("LTC_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        c = ctypes
        L.ltco_elem_bytes.argtypes = [c.c_int]
        L.ltco_reorder.argtypes = [c.c_int, c.c_uint32]
        L.ltco_reorder.restype = c.c_uint32
        L.ltco_unreorder.argtypes = [c.c_int, c.c_uint32]
        L.ltco_unreorder.restype = c.c_uint32
        L.ltco_chunk_stream.argtypes = [u8p, c.c_uint64, c.c_int, c.c_uint32,
                                        c.c_uint64, c.c_int, u8p]
        L.ltco_chunk_stream.restype = c.c_uint64
        L.ltco_histogram.argtypes = [u8p, c.c_uint64, u64p]
        L.ltco_normalize.argtypes = [u64p, u16p]
        L.ltco_p_max.argtypes = [c.c_uint64, c.c_double]
        L.ltco_p_max.restype = c.c_uint64
        L.ltco_rans_encode.argtypes = [u8p, c.c_uint64, u16p, u32p, u16p,
                                       c.c_uint64, u64p]
        L.ltco_rans_decode.argtypes = [u16p, c.c_uint64, u32p, u16p,
                                       c.c_uint64, u8p]
        L.ltco_compress_bound.argtypes = [c.c_uint64, c.c_int, c.c_uint32]
        L.ltco_compress_bound.restype = c.c_uint64
        L.ltco_compress.argtypes = [u8p, c.c_uint64, c.c_int, c.c_uint32,
                                    c.c_double, u8p, c.c_uint64, u64p, c.c_int]
        L.ltco_compress_bound_ex.argtypes = [c.c_uint64, c.c_int, c.c_uint32, c.c_uint32]
        L.ltco_compress_bound_ex.restype = c.c_uint64
        L.ltco_compress_ex.argtypes = [u8p, c.c_uint64, c.c_int, c.c_uint32, c.c_double,
                                       c.c_uint32, u8p, c.c_uint64, u64p, c.c_int]
        L.ltco_compress_delta.argtypes = [u8p, u8p, c.c_uint64, c.c_int, c.c_uint32, c.c_double,
                                          c.c_uint32, u8p, c.c_uint64, u64p, c.c_int]
        L.ltco_decompress_delta.argtypes = [u8p, c.c_uint64, u8p, u8p, c.c_uint64, u64p, c.c_int]
        L.ltco_encode_chunk.argtypes = [u8p, c.c_uint64, c.c_int, c.c_uint32,
                                        c.c_double, c.c_uint64, u8p, u8p, u32p,
                                        u8p, c.c_uint64, u64p]
        L.ltco_decompress.argtypes = [u8p, c.c_uint64, u8p, c.c_uint64, u64p,
                                      c.c_int]
        L.ltco_crc32.argtypes = [u8p, c.c_uint64]
        L.ltco_crc32.restype = c.c_uint32
        L.ltco_crc32_chunks.argtypes = [u8p, c.c_uint64, c.c_uint32, u32p]
        _lib = L
    return _lib


def _as_bytes(a):
    a = np.ascontiguousarray(a)
    return a.reshape(-1).view(np.uint8)


def reorder(dtype, x):
    return lib().ltco_reorder(dtype, int(x))


def unreorder(dtype, y):
    return lib().ltco_unreorder(dtype, int(y))


def chunk_stream(src, dtype, chunk_bytes, c, k):
    b = _as_bytes(src)
    out = np.zeros(chunk_bytes, dtype=np.uint8)
    n = lib().ltco_chunk_stream(_u8p(b), b.size, dtype, chunk_bytes, c, k, _u8p(out))
    return out[:n].copy()


def histogram(sym):
    s = np.ascontiguousarray(sym, dtype=np.uint8)
    h = np.zeros(256, dtype=np.uint64)
    lib().ltco_histogram(_u8p(s), s.size, h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    return h


def normalize(h):
    h = np.ascontiguousarray(h, dtype=np.uint64)
    f = np.zeros(256, dtype=np.uint16)
    rc = lib().ltco_normalize(h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                              f.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)))
    if rc:
        raise ValueError(f"normalize: status {rc}")
    return f


def p_max(n, theta):
    return lib().ltco_p_max(n, theta)


def rans_encode(sym, f):
    s = np.ascontiguousarray(sym, dtype=np.uint8)
    f = np.ascontiguousarray(f, dtype=np.uint16)
    states = np.zeros(64, dtype=np.uint32)
    words = np.zeros(max(1, s.size), dtype=np.uint16)
    nw = ctypes.c_uint64(0)
    rc = lib().ltco_rans_encode(_u8p(s), s.size,
                                f.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                states.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                words.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                words.size, ctypes.byref(nw))
    if rc:
        raise ValueError(f"rans_encode: status {rc}")
    return states, words[: nw.value].copy()


def rans_decode(words, states, f, n):
    w = np.ascontiguousarray(words, dtype=np.uint16)
    st = np.ascontiguousarray(states, dtype=np.uint32)
    f = np.ascontiguousarray(f, dtype=np.uint16)
    out = np.zeros(max(1, n), dtype=np.uint8)
    rc = lib().ltco_rans_decode(w.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), w.size,
                                st.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                f.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                                n, _u8p(out))
    return rc, out[:n].copy()


def compress_bound(nbytes, dtype, chunk_bytes=131072, shared_tables=False):
    return lib().ltco_compress_bound_ex(nbytes, dtype, chunk_bytes,
                                        FLAG_SHARED_TABLES if shared_tables else 0)


def _flags(shared_tables, top_last):
    return (FLAG_SHARED_TABLES if shared_tables else 0) | (FLAG_TOP_LAST if top_last else 0)


def compress(src, dtype, chunk_bytes=131072, threshold=0.95, nthreads=None, shared_tables=False,
             top_last=False):
    """Blob (np.uint8) of the bytes of `src` read as `dtype` (a code);
    shared_tables: format v2 (one frequency table per stream index);
    top_last: the top stream of every chunk placed after all other payloads."""
    b = _as_bytes(src)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    cap = max(64, compress_bound(b.size, dtype, chunk_bytes, shared_tables))
    blob = np.zeros(cap, dtype=np.uint8)
    nb = ctypes.c_uint64(0)
    rc = lib().ltco_compress_ex(_u8p(b), b.size, dtype, chunk_bytes, threshold,
                                _flags(shared_tables, top_last),
                                _u8p(blob), blob.size, ctypes.byref(nb), int(nthreads))
    if rc:
        raise ValueError(f"oracle compress: status {rc}")
    return blob[: nb.value].copy()


def compress_delta(src, base, dtype, chunk_bytes=131072, threshold=0.95, nthreads=None,
                   shared_tables=False, top_last=False):
    """Blob of src XOR base (same byte size), with ZipNN's zero-run rule."""
    b = _as_bytes(src)
    bb = _as_bytes(base)
    if bb.size != b.size:
        raise ValueError("base must have the input's size")
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    cap = max(64, compress_bound(b.size, dtype, chunk_bytes, shared_tables))
    blob = np.zeros(cap, dtype=np.uint8)
    nb = ctypes.c_uint64(0)
    rc = lib().ltco_compress_delta(_u8p(b), _u8p(bb), b.size, dtype, chunk_bytes, threshold,
                                   _flags(shared_tables, top_last),
                                   _u8p(blob), blob.size, ctypes.byref(nb), int(nthreads))
    if rc:
        raise ValueError(f"oracle compress_delta: status {rc}")
    return blob[: nb.value].copy()


def decompress_delta(blob, base, nthreads=None):
    """(status, decoded bytes) of a delta blob given its base."""
    bl = np.ascontiguousarray(blob, dtype=np.uint8)
    bb = _as_bytes(base)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    capacity = int.from_bytes(bytes(bl[8:16]), "little") if bl.size >= 16 else 0
    dst = np.zeros(max(1, capacity), dtype=np.uint8)
    if bb.size < capacity:
        return ERR_INVALID_ARGUMENT, None
    nout = ctypes.c_uint64(0)
    rc = lib().ltco_decompress_delta(_u8p(bl), bl.size, _u8p(bb), _u8p(dst), capacity,
                                     ctypes.byref(nout), int(nthreads))
    if rc:
        return rc, None
    return rc, dst[: nout.value].copy()


def encode_chunk(src, dtype, chunk_bytes, threshold, c):
    """(modes, cvals, sizes, padded payload bytes) of chunk c alone."""
    b = _as_bytes(src)
    e = ELEM_BYTES[dtype]
    modes = np.zeros(e, dtype=np.uint8)
    cvals = np.zeros(e, dtype=np.uint8)
    sizes = np.zeros(e, dtype=np.uint32)
    out = np.zeros(chunk_bytes + 16 * e + 64, dtype=np.uint8)
    nout = ctypes.c_uint64(0)
    rc = lib().ltco_encode_chunk(_u8p(b), b.size, dtype, chunk_bytes, threshold, c,
                                 _u8p(modes), _u8p(cvals),
                                 sizes.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                                 _u8p(out), out.size, ctypes.byref(nout))
    if rc:
        raise ValueError(f"oracle encode_chunk: status {rc}")
    return modes, cvals, sizes, out[: nout.value].copy()


def decompress(blob, capacity=None, nthreads=None):
    """(status, decoded bytes as np.uint8)."""
    bl = np.ascontiguousarray(blob, dtype=np.uint8)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    if capacity is None:
        capacity = int.from_bytes(bytes(bl[8:16]), "little") if bl.size >= 16 else 0
    dst = np.zeros(max(1, capacity), dtype=np.uint8)
    nout = ctypes.c_uint64(0)
    rc = lib().ltco_decompress(_u8p(bl), bl.size, _u8p(dst), capacity,
                               ctypes.byref(nout), int(nthreads))
    if rc:
        return rc, None
    return rc, dst[: nout.value].copy()


def crc32(data):
    b = _as_bytes(data)
    return lib().ltco_crc32(_u8p(b), b.size)


def crc32_chunks(data, chunk_bytes=16384):
    b = _as_bytes(data)
    count = (b.size + chunk_bytes - 1) // chunk_bytes
    out = np.zeros(max(1, count), dtype=np.uint32)
    rc = lib().ltco_crc32_chunks(_u8p(b), b.size, chunk_bytes,
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)))
    if rc:
        raise ValueError(f"oracle crc32_chunks: status {rc}")
    return out[:count].copy()
