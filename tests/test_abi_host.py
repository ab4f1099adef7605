"""Host-side checks of the C ABI that need no GPU: the shared library loads,
exports every entry point include/ltc.h declares, and its host logic (size
bounds, header parsing, statistics, argument validation) agrees with the
format the oracle writes."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ltc = pytest.importorskip("lossless_tensor_compression_amd")


def _lib():
    if not os.path.exists(ltc.LIB_PATH):
        import lossless_tensor_compression_amd.build as b
        b.build()
    return ltc.lib()


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "ltc.h")).read()
    declared = set(re.findall(r"\b(ltc_[a-z0-9_]+)\s*\(", header))
    assert {"ltc_compress", "ltc_decompress", "ltc_crc32_chunks"} <= declared
    L = ctypes.CDLL(ltc.LIB_PATH if os.path.exists(ltc.LIB_PATH) else _lib()._name)
    missing = [s for s in sorted(declared) if not hasattr(L, s)]
    assert not missing, missing


@pytest.mark.parametrize("dtype,chunk", [(0, 8), (1, 131072), (2, 4096), (3, 131072), (3, 24)])
@pytest.mark.parametrize("nbytes", [0, 4, 8, 100, 131072, 131072 * 3 + 20])
def test_bound_matches_oracle(dtype, chunk, nbytes):
    _lib()
    e = oracle.ELEM_BYTES[dtype]
    nbytes -= nbytes % e
    assert ltc.compress_bound(nbytes, dtype, chunk) == oracle.compress_bound(nbytes, dtype, chunk)


def test_bound_rejects_bad_args():
    _lib()
    assert ltc.compress_bound(10, 9, 131072) == 0
    assert ltc.compress_bound(3, 1, 131072) == 0
    assert ltc.compress_bound(16, 0, 12) == 0
    assert ltc.compress_bound(16, 0, (1 << 24) + 8) == 0


def test_blob_info_and_stats_on_oracle_blob():
    _lib()
    x = workloads.c1()
    blob = oracle.compress(x, 1)
    info = ltc.blob_info(bytes(blob[:64]))
    assert info["dtype"] == 1 and info["elem_bytes"] == 2 and info["nbytes"] == x.nbytes
    assert info["chunk_bytes"] == 131072 and info["nchunks"] == 16
    assert info["blob_nbytes"] == blob.size and info["payload_base"] == 64 + 16 * 32
    st = ctypes.create_string_buffer(bytes(blob[:info["payload_base"]]))
    stats = ltc.Stats()
    assert ltc.lib().ltc_blob_stats(st.raw, info["payload_base"], ctypes.byref(stats)) == 0
    assert stats.mode_count[0][0] == 16 and stats.mode_count[1][1] == 16
    assert stats.payload_bytes[0] == stats.stream_bytes[0] == 16 * 65536
    assert 0.30 < stats.payload_bytes[1] / stats.stream_bytes[1] < 0.35


def test_blob_info_top_last():
    _lib()
    x = workloads.c1()
    blob = oracle.compress(x, 1, top_last=True)
    info = ltc.blob_info(bytes(blob[:64]))
    assert info["flags"] == 8 and info["version"] == 1 and info["blob_nbytes"] == blob.size
    v2 = oracle.compress(x, 1, shared_tables=True, top_last=True)
    assert ltc.blob_info(bytes(v2[:64]))["flags"] == 9


def _info_rc(hdr):
    out = ltc.Info()
    return ltc.lib().ltc_blob_info(bytes(hdr), len(hdr), ctypes.byref(out))


def test_blob_info_errors_match_oracle():
    _lib()
    blob = oracle.compress(workloads.c1()[:5000], 1, 1024)
    assert _info_rc(blob[:64]) == 0
    cases = []
    for pos, val in ((0, 0x4D), (4, 2), (4, 3), (6, 7), (7, 4), (24, 32), (26, 11), (27, 1),
                     (27, 9), (27, 16), (28, 1), (50, 1), (16, 0), (20, 99), (40, 0)):
        b = blob.copy()
        b[pos] = val
        cases.append(b)
    for b in cases:
        want = oracle.decompress(b)[0]
        got = _info_rc(b[:64])
        assert got == want, (got, want)
    assert _info_rc(blob[:63]) == ltc.lib().ltc_blob_info(bytes(blob[:63]), 63, ctypes.byref(ltc.Info()))
    assert _info_rc(blob[:40]) == -5
    # a 64-byte blob claiming N = 2^64 - 8 in K = 0 chunks: ceil(N / C) must
    # not wrap around to K (otherwise the header is consistent: empty
    # directory, payload_base = blob_nbytes = 64)
    b = blob[:64].copy()
    b[8:16] = np.frombuffer((2**64 - 8).to_bytes(8, "little"), dtype=np.uint8)
    b[20:24] = 0
    b[32:40] = np.frombuffer((64).to_bytes(8, "little"), dtype=np.uint8)
    b[40:48] = np.frombuffer((64).to_bytes(8, "little"), dtype=np.uint8)
    assert _info_rc(b) == oracle.decompress(b, capacity=0)[0] == -5


def test_argument_errors_before_any_launch():
    L = _lib()
    null = ctypes.c_void_p(0)
    ws = ctypes.c_uint64(0)
    assert L.ltc_compress_workspace_size(10, 9, 131072, ctypes.byref(ws)) == -2
    assert L.ltc_compress_workspace_size(3, 1, 131072, ctypes.byref(ws)) == -1
    assert L.ltc_compress_workspace_size(1 << 20, 1, 131072, ctypes.byref(ws)) == 0 and ws.value > 0
    # bad dtype / size / chunk / threshold are rejected on the host
    fake = ctypes.c_void_p(1 << 20)
    assert L.ltc_compress(fake, 16, 9, 131072, 0.95, fake, 1 << 20, fake, fake, 1 << 30, null) == -2
    assert L.ltc_compress(fake, 15, 1, 131072, 0.95, fake, 1 << 20, fake, fake, 1 << 30, null) == -1
    assert L.ltc_compress(fake, 16, 1, 12, 0.95, fake, 1 << 20, fake, fake, 1 << 30, null) == -1
    assert L.ltc_compress(fake, 16, 1, 131072, 0.0, fake, 1 << 20, fake, fake, 1 << 30, null) == -1
    assert L.ltc_compress(fake, 16, 1, 131072, 1.5, fake, 1 << 20, fake, fake, 1 << 30, null) == -1
    assert L.ltc_compress(fake, 16, 1, 131072, 0.95, fake, 16, fake, fake, 1 << 30, null) == -6
    assert L.ltc_compress(fake, 16, 1, 131072, 0.95, fake, 1 << 20, fake, fake, 16, null) == -7
    assert L.ltc_crc32_chunks(fake, 100, 0, fake, null) == -1
    assert L.ltc_crc32_chunks(fake, 0, 16384, fake, null) == 0
    # compress_with_crc32: checksum chunk 0, short or misaligned checksum array
    cwc = L.ltc_compress_with_crc32
    cwc.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32, ctypes.c_double,
                    ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p,
                    ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    bound = L.ltc_compress_bound(4096, 1, 131072)
    need = (bound + 1023) // 1024
    assert cwc(fake, 4096, 1, 131072, 0.95, fake, bound, fake, 0, fake, 99, fake, 1 << 30, null) == -1
    assert cwc(fake, 4096, 1, 131072, 0.95, fake, bound, fake, 1024, fake, need - 1, fake, 1 << 30,
               null) == -6
    assert cwc(fake, 4096, 1, 131072, 0.95, fake, bound, fake, 1024, ctypes.c_void_p((1 << 20) + 2),
               need, fake, 1 << 30, null) == -1
    assert cwc(fake, 4096, 9, 131072, 0.95, fake, bound, fake, 1024, fake, need, fake, 1 << 30, null) == -2
    assert cwc(fake, 4096, 1, 131072, 0.95, fake, bound, fake, 1024, fake, need, fake, 16, null) == -7


def test_noalloc_limits_before_any_launch():
    """ltc_compress_noalloc checks its arguments and the size of its fixed
    workspace on the host, before touching the device: an input whose
    workspace exceeds LTC_NOALLOC_SCRATCH_BYTES is refused with WORKSPACE."""
    L = _lib()
    null = ctypes.c_void_p(0)
    fake = ctypes.c_void_p(1 << 20)
    ws = ctypes.c_uint64(0)
    limit = ltc.NOALLOC_SCRATCH_BYTES
    # the largest BF16 input (whole chunks) whose workspace fits, and one chunk more
    per = 1
    while True:
        assert L.ltc_compress_workspace_size(per * 131072, 1, 131072, ctypes.byref(ws)) == 0
        if ws.value > limit:
            break
        per += 1
    assert per > 400  # about 60 MB of BF16
    big = per * 131072
    bound = L.ltc_compress_bound(big, 1, 131072)
    assert L.ltc_compress_noalloc(fake, big, 1, 131072, 0.95, fake, bound, fake, null) == -7
    assert L.ltc_compress_noalloc(fake, 1 << 40, 1, 131072, 0.95, fake, 1 << 41, fake, null) == -7
    assert L.ltc_compress_noalloc(fake, 16, 9, 131072, 0.95, fake, 1 << 20, fake, null) == -2
    assert L.ltc_compress_noalloc(fake, 15, 1, 131072, 0.95, fake, 1 << 20, fake, null) == -1
    assert L.ltc_compress_noalloc(fake, 16, 1, 12, 0.95, fake, 1 << 20, fake, null) == -1


def test_stream_and_layout_flags_do_not_change_the_bound():
    _lib()
    for dtype in (0, 1, 3):
        n = 131072 * 5 + 8
        base = ltc.lib().ltc_compress_bound_ex(n, dtype, 131072, 0)
        assert base == ltc.compress_bound(n, dtype)
        assert ltc.lib().ltc_compress_bound_ex(n, dtype, 131072, ltc.FLAG_CALLER_STREAM_ONLY) == base
        assert ltc.lib().ltc_compress_bound_ex(n, dtype, 131072, ltc.FLAG_TOP_LAST) == base
        assert ltc.lib().ltc_compress_bound_ex(n, dtype, 131072, ltc.FLAG_PLACE_NO_WAIT) == base
        assert ltc.lib().ltc_compress_bound_ex(n, dtype, 131072, 32) == 0  # unknown flag
