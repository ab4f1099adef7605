"""MI355X-native ZipNN-style lossless compression of model-weight tensors.

A thin ctypes binding over libltc.so (HIP kernels for gfx950 behind the C ABI
in include/ltc.h).  Every step of compression, decompression and checksum
runs in the library's kernels; this module only marshals torch tensors
(device memory and the current stream) to the C entry points.  There is no
CPU fallback: without the built library, or without a GPU, calls raise.

API (names as in cuZipNN 0.1.0, "API", and the C ABI):
  compress(t, chunk_bytes=131072, passthrough_threshold=0.95) -> uint8 blob
  decompress(blob, shape=None) -> tensor of the recorded dtype
  crc32_chunks(t, chunk_bytes=16384) -> int32 tensor holding CRC-32 bits
  compress_with_crc32(t, ..., checksum_chunk_bytes=16384) -> (blob, CRC-32 of
      the blob's chunks), the checksums computed while the blob is written
  compress_to_host(t) -> pinned CPU blob; decompress_from_host(cpu_blob) ->
      GPU tensor (copies of chunk groups overlapped with their decoding)
  compress_batch / decompress_batch for many tensors in one launch sequence
  compress_delta(t, base) / decompress_delta(blob, base): XOR deltas against
      a base tensor, zero-run coded where the delta is mostly zero bytes
  blob_info / blob_stats for host-side inspection of a blob's header
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libltc.so")

U8, BF16, FP16, FP32 = 0, 1, 2, 3
DTYPE_CODE = {torch.uint8: U8, torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}
ERRORS = {0: "OK", -1: "INVALID_ARGUMENT", -2: "UNSUPPORTED_DTYPE", -3: "BAD_MAGIC",
          -4: "BAD_VERSION", -5: "CORRUPT", -6: "CAPACITY", -7: "WORKSPACE", -8: "HIP"}
BATCH_MAX = 32
DEFAULT_CHUNK_BYTES = 131072
DEFAULT_THRESHOLD = 0.95
DEFAULT_CRC_CHUNK_BYTES = 16384


class LTCError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({code})")
        self.code = code


class Info(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("elem_bytes", ctypes.c_uint32),
                ("nbytes", ctypes.c_uint64), ("chunk_bytes", ctypes.c_uint32),
                ("nchunks", ctypes.c_uint32), ("blob_nbytes", ctypes.c_uint64),
                ("payload_base", ctypes.c_uint64), ("version", ctypes.c_uint32),
                ("flags", ctypes.c_uint32)]


class Stats(ctypes.Structure):
    _fields_ = [("elem_bytes", ctypes.c_uint32), ("nbytes", ctypes.c_uint64),
                ("blob_nbytes", ctypes.c_uint64),
                ("mode_count", (ctypes.c_uint64 * 4) * 4),
                ("payload_bytes", ctypes.c_uint64 * 4),
                ("stream_bytes", ctypes.c_uint64 * 4)]


_lib = None


def lib():
    """The loaded libltc.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python lossless_tensor_compression_amd/build.py` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, u64, u32, i32, dbl = (ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_int, ctypes.c_double)
        pvp = ctypes.POINTER(ctypes.c_void_p)
        pu64 = ctypes.POINTER(ctypes.c_uint64)
        L.ltc_elem_bytes.argtypes = [i32]
        L.ltc_elem_bytes.restype = u32
        L.ltc_compress_bound.argtypes = [u64, i32, u32]
        L.ltc_compress_bound.restype = u64
        L.ltc_compress_workspace_size.argtypes = [u64, i32, u32, pu64]
        L.ltc_compress_batch_workspace_size.argtypes = [i32, pu64, i32, u32, pu64]
        L.ltc_compress.argtypes = [vp, u64, i32, u32, dbl, vp, u64, vp, vp, u64, vp]
        L.ltc_compress_noalloc.argtypes = [vp, u64, i32, u32, dbl, vp, u64, vp, vp]
        L.ltc_compress_batch.argtypes = [i32, pvp, pu64, i32, u32, dbl, pvp, pu64, vp, vp, u64, vp]
        L.ltc_compress_batch_prof.argtypes = [i32, pvp, pu64, i32, u32, dbl, pvp, pu64, vp, vp,
                                              u64, vp, pvp]
        L.ltc_compress_with_crc32.argtypes = [vp, u64, i32, u32, dbl, vp, u64, vp, u32, vp, u64,
                                              vp, u64, vp]
        L.ltc_compress_bound_ex.argtypes = [u64, i32, u32, u32]
        L.ltc_compress_bound_ex.restype = u64
        L.ltc_compress_batch_ex.argtypes = [i32, pvp, pu64, i32, u32, dbl, u32, pvp, pvp, pu64, vp,
                                            u32, pvp, pu64, vp, u64, vp, pvp]
        L.ltc_compress_delta.argtypes = [vp, vp, u64, i32, u32, dbl, u32, vp, u64, vp, vp, u64, vp]
        L.ltc_decompress_delta_workspace_size.argtypes = [i32, pvp, pu64]
        L.ltc_decompress_delta_batch.argtypes = [i32, pvp, pvp, pu64, pvp, pvp, pu64, vp, vp, u64, vp]
        L.ltc_decompress_delta.argtypes = [ctypes.c_char_p, vp, u64, vp, vp, u64, vp, vp, u64, vp]
        L.ltc_compress_batch_with_crc32.argtypes = [i32, pvp, pu64, i32, u32, dbl, pvp, pu64, vp,
                                                    u32, pvp, pu64, vp, u64, vp]
        L.ltc_compress_batch_with_crc32_prof.argtypes = [i32, pvp, pu64, i32, u32, dbl, pvp, pu64,
                                                         vp, u32, pvp, pu64, vp, u64, vp, pvp]
        L.ltc_blob_info.argtypes = [ctypes.c_char_p, u64, ctypes.POINTER(Info)]
        L.ltc_decompress.argtypes = [ctypes.c_char_p, vp, u64, vp, u64, vp, vp]
        L.ltc_decompress_batch.argtypes = [i32, pvp, pvp, pu64, pvp, pu64, vp, vp]
        L.ltc_decompress_batch_prof.argtypes = [i32, pvp, pvp, pu64, pvp, pu64, vp, vp, pvp]
        L.ltc_decompress_from_host.argtypes = [vp, u64, vp, u64, vp, vp, u64, vp]
        L.ltc_decompress_batch_from_host.argtypes = [i32, pvp, pu64, pvp, pu64, vp, pvp, pu64, vp]
        L.ltc_crc32_chunks.argtypes = [vp, u64, u32, vp, vp]
        L.ltc_crc32_chunks_batch.argtypes = [i32, pvp, pu64, u32, pvp, vp]
        L.ltc_blob_stats.argtypes = [ctypes.c_char_p, u64, ctypes.POINTER(Stats)]
        for name in ("ltc_compress_workspace_size", "ltc_compress_batch_workspace_size",
                     "ltc_compress", "ltc_compress_noalloc", "ltc_compress_batch",
                     "ltc_compress_batch_prof",
                     "ltc_compress_with_crc32", "ltc_compress_batch_with_crc32", "ltc_compress_batch_ex",
                     "ltc_compress_batch_with_crc32_prof",
                     "ltc_blob_info", "ltc_decompress", "ltc_decompress_batch",
                     "ltc_decompress_batch_prof", "ltc_decompress_from_host",
                     "ltc_decompress_batch_from_host", "ltc_crc32_chunks", "ltc_crc32_chunks_batch",
                     "ltc_blob_stats", "ltc_compress_delta", "ltc_decompress_delta_workspace_size",
                     "ltc_decompress_delta_batch", "ltc_decompress_delta"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise LTCError(rc, what)


class Prepared:
    """One C ABI call with its arguments marshalled once, for loops that
    repeat the same call (the host then pays only the foreign call).  keep:
    objects the marshalled pointers refer to."""

    def __init__(self, fn, args, what, keep=None):
        self._fn, self._args, self._what, self._keep = fn, args, what, keep

    def __call__(self):
        _check(self._fn(*self._args), self._what)


def _run(fn, args, what, prepare, keep=None):
    if prepare:
        return Prepared(fn, args, what, keep)
    _check(fn(*args), what)
    return None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptrs(seq):
    return (ctypes.c_void_p * len(seq))(*[ctypes.c_void_p(p) for p in seq])


def _u64s(seq):
    return (ctypes.c_uint64 * len(seq))(*seq)


def _flat_bytes(t):
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU")
    if t.dtype not in DTYPE_CODE:
        raise LTCError(-2, f"dtype {t.dtype}")
    return t.contiguous()


FLAG_SHARED_TABLES = 1  # format v2: one frequency table per stream index
FLAG_DELTA = 2          # header flag: the blob codes src XOR base
FLAG_CALLER_STREAM_ONLY = 4  # compress flag: every kernel on the caller's stream
FLAG_TOP_LAST = 8       # compress and header flag: top-stream payloads after all others
FLAG_PLACE_NO_WAIT = 16  # compress flag, top-last: placing encoder waves never wait (tests)
NOALLOC_SCRATCH_BYTES = 64 << 20  # workspace limit of ltc_compress_noalloc


def _flags(shared_tables, top_last):
    return (FLAG_SHARED_TABLES if shared_tables else 0) | (FLAG_TOP_LAST if top_last else 0)


def compress_bound(nbytes, dtype_code, chunk_bytes=DEFAULT_CHUNK_BYTES, shared_tables=False):
    return int(lib().ltc_compress_bound_ex(nbytes, dtype_code, chunk_bytes,
                                           FLAG_SHARED_TABLES if shared_tables else 0))


def workspace_size(nbytes_list, dtype_code, chunk_bytes=DEFAULT_CHUNK_BYTES):
    out = ctypes.c_uint64(0)
    _check(lib().ltc_compress_batch_workspace_size(len(nbytes_list), _u64s(nbytes_list), dtype_code,
                                                   chunk_bytes, ctypes.byref(out)), "workspace size")
    return out.value


def compress_raw(src_ptrs, nbytes, dtype_code, chunk_bytes, threshold, blob_ptrs, caps,
                 nbytes_out_ptr, ws_ptr, ws_nbytes, stream=None, events=None):
    """Pointer-level batch compress on `stream` (no allocation, no sync)."""
    count = len(src_ptrs)
    args = [count, _ptrs(src_ptrs), _u64s(nbytes), dtype_code, chunk_bytes, threshold,
            _ptrs(blob_ptrs), _u64s(caps), ctypes.c_void_p(nbytes_out_ptr),
            ctypes.c_void_p(ws_ptr), ws_nbytes, _stream(stream)]
    if events is None:
        _check(lib().ltc_compress_batch(*args), "compress")
    else:
        _check(lib().ltc_compress_batch_prof(*args, _ptrs(events)), "compress")


def compress_noalloc_raw(src_ptr, nbytes, dtype_code, chunk_bytes, threshold, blob_ptr, cap,
                         nbytes_out_ptr, stream=None):
    """Pointer-level ltc_compress_noalloc on `stream`: the workspace is the
    library's own device array (inputs up to NOALLOC_SCRATCH_BYTES of
    workspace), nothing is allocated."""
    _check(lib().ltc_compress_noalloc(ctypes.c_void_p(src_ptr), nbytes, dtype_code, chunk_bytes,
                                      threshold, ctypes.c_void_p(blob_ptr), cap,
                                      ctypes.c_void_p(nbytes_out_ptr), _stream(stream)),
           "compress_noalloc")


def compress_ex_raw(src_ptrs, nbytes, dtype_code, chunk_bytes, threshold, flags, blob_ptrs, caps,
                    nbytes_out_ptr, ws_ptr, ws_nbytes, crc_chunk_bytes=0, crc_ptrs=None,
                    crc_caps=None, stream=None, events=None, base_ptrs=None, prepare=False):
    """Pointer-level ltc_compress_batch_ex: format flags, optional checksums
    (crc_chunk_bytes > 0), optional events (5, or 6 with checksums) and
    optional delta bases (XOR deltas).  prepare: return a Prepared call
    instead of calling."""
    count = len(src_ptrs)
    crc_ptrs = crc_ptrs or [0] * count
    crc_caps = crc_caps or [0] * count
    ev = _ptrs(events) if events is not None else None
    bases = _ptrs(base_ptrs) if base_ptrs is not None else None
    args = (count, _ptrs(src_ptrs), _u64s(nbytes), dtype_code, chunk_bytes, threshold, flags, bases,
            _ptrs(blob_ptrs), _u64s(caps), ctypes.c_void_p(nbytes_out_ptr), crc_chunk_bytes, _ptrs(crc_ptrs),
            _u64s(crc_caps), ctypes.c_void_p(ws_ptr), ws_nbytes, _stream(stream), ev)
    return _run(lib().ltc_compress_batch_ex, args, "compress", prepare)


def compress_crc32_raw(src_ptrs, nbytes, dtype_code, chunk_bytes, threshold, blob_ptrs, caps,
                       nbytes_out_ptr, crc_chunk_bytes, crc_ptrs, crc_caps, ws_ptr, ws_nbytes,
                       stream=None, events=None):
    """Pointer-level batch compress plus CRC-32 of each blob (6 events with
    `events`)."""
    count = len(src_ptrs)
    args = [count, _ptrs(src_ptrs), _u64s(nbytes), dtype_code, chunk_bytes, threshold,
            _ptrs(blob_ptrs), _u64s(caps), ctypes.c_void_p(nbytes_out_ptr), crc_chunk_bytes,
            _ptrs(crc_ptrs), _u64s(crc_caps), ctypes.c_void_p(ws_ptr), ws_nbytes, _stream(stream)]
    if events is None:
        _check(lib().ltc_compress_batch_with_crc32(*args), "compress_with_crc32")
    else:
        _check(lib().ltc_compress_batch_with_crc32_prof(*args, _ptrs(events)), "compress_with_crc32")


def decompress_raw(headers, blob_ptrs, blob_nbytes, dst_ptrs, caps, status_ptr, stream=None,
                   events=None, prepare=False):
    """Pointer-level batch decompress on `stream`; headers are 64-byte host
    bytes.  prepare: return a Prepared call instead of calling."""
    count = len(blob_ptrs)
    hdr = (ctypes.c_void_p * count)(*[ctypes.cast(ctypes.c_char_p(h), ctypes.c_void_p) for h in headers])
    args = [count, hdr, _ptrs(blob_ptrs), _u64s(blob_nbytes), _ptrs(dst_ptrs), _u64s(caps),
            ctypes.c_void_p(status_ptr), _stream(stream)]
    if events is None:
        return _run(lib().ltc_decompress_batch, args, "decompress", prepare, keep=list(headers))
    return _run(lib().ltc_decompress_batch_prof, args + [_ptrs(events)], "decompress", prepare,
                keep=list(headers))


def compress_batch(tensors, chunk_bytes=DEFAULT_CHUNK_BYTES,
                   passthrough_threshold=DEFAULT_THRESHOLD, shared_tables=False, top_last=False):
    """Blobs (uint8 GPU tensors) for up to 32 tensors of one dtype;
    shared_tables: format v2 (one frequency table per stream index);
    top_last: the top-last payload layout (LTC_FLAG_TOP_LAST)."""
    return _compress_batch(tensors, None, chunk_bytes, passthrough_threshold, shared_tables, top_last)


def compress_batch_delta(tensors, bases, chunk_bytes=DEFAULT_CHUNK_BYTES,
                         passthrough_threshold=DEFAULT_THRESHOLD, shared_tables=False, top_last=False):
    """XOR-delta blobs of up to 32 tensors against their bases (same dtype
    and size each): ZipNN's delta compression of a fine-tuned model against
    its base model."""
    if len(bases) != len(tensors):
        raise ValueError("one base per tensor")
    return _compress_batch(tensors, bases, chunk_bytes, passthrough_threshold, shared_tables, top_last)


def compress_delta(t, base, chunk_bytes=DEFAULT_CHUNK_BYTES, passthrough_threshold=DEFAULT_THRESHOLD,
                   shared_tables=False, top_last=False):
    """XOR-delta blob of a GPU tensor against a base of the same dtype and size."""
    return compress_batch_delta([t], [base], chunk_bytes, passthrough_threshold, shared_tables,
                                top_last)[0]


def _compress_batch(tensors, bases, chunk_bytes, passthrough_threshold, shared_tables, top_last=False):
    if not 1 <= len(tensors) <= BATCH_MAX:
        raise ValueError(f"1..{BATCH_MAX} tensors per batch")
    ts = [_flat_bytes(t) for t in tensors]
    code = DTYPE_CODE[ts[0].dtype]
    if any(DTYPE_CODE[t.dtype] != code for t in ts):
        raise ValueError("one dtype per batch")
    bs = None
    if bases is not None:
        bs = [_flat_bytes(b) for b in bases]
        if any(b.dtype != t.dtype or b.numel() != t.numel() or b.device != t.device
               for b, t in zip(bs, ts)):
            raise ValueError("a base must match its tensor's dtype, size and device")
    dev = ts[0].device
    nbytes = [t.numel() * t.element_size() for t in ts]
    caps = [compress_bound(n, code, chunk_bytes, shared_tables) for n in nbytes]
    if any(c == 0 for c in caps):
        raise LTCError(-1, "compress_bound")
    blobs = [torch.empty(c, dtype=torch.uint8, device=dev) for c in caps]
    ws_n = workspace_size(nbytes, code, chunk_bytes)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
    sizes = torch.zeros(len(ts), dtype=torch.int64, device=dev)
    compress_ex_raw([t.data_ptr() for t in ts], nbytes, code, chunk_bytes, passthrough_threshold,
                    _flags(shared_tables, top_last), [b.data_ptr() for b in blobs], caps,
                    sizes.data_ptr(), ws.data_ptr(), ws.numel(),
                    base_ptrs=[b.data_ptr() for b in bs] if bs is not None else None)
    host_sizes = sizes.cpu().tolist()
    return [b[:s] for b, s in zip(blobs, host_sizes)]


def compress_batch_with_crc32(tensors, chunk_bytes=DEFAULT_CHUNK_BYTES,
                              passthrough_threshold=DEFAULT_THRESHOLD,
                              checksum_chunk_bytes=DEFAULT_CRC_CHUNK_BYTES, shared_tables=False,
                              top_last=False):
    """(blobs, checksums): the blobs of compress_batch and, per blob, one
    CRC-32 per checksum_chunk_bytes bytes of it (int32 GPU tensors holding
    the CRC bits)."""
    if not 1 <= len(tensors) <= BATCH_MAX:
        raise ValueError(f"1..{BATCH_MAX} tensors per batch")
    ts = [_flat_bytes(t) for t in tensors]
    code = DTYPE_CODE[ts[0].dtype]
    if any(DTYPE_CODE[t.dtype] != code for t in ts):
        raise ValueError("one dtype per batch")
    if checksum_chunk_bytes <= 0:
        raise LTCError(-1, "checksum_chunk_bytes")
    dev = ts[0].device
    nbytes = [t.numel() * t.element_size() for t in ts]
    caps = [compress_bound(n, code, chunk_bytes, shared_tables) for n in nbytes]
    if any(c == 0 for c in caps):
        raise LTCError(-1, "compress_bound")
    blobs = [torch.empty(c, dtype=torch.uint8, device=dev) for c in caps]
    ccaps = [(c + checksum_chunk_bytes - 1) // checksum_chunk_bytes for c in caps]
    crcs = [torch.empty(n, dtype=torch.int32, device=dev) for n in ccaps]
    ws_n = workspace_size(nbytes, code, chunk_bytes)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
    sizes = torch.zeros(len(ts), dtype=torch.int64, device=dev)
    compress_ex_raw([t.data_ptr() for t in ts], nbytes, code, chunk_bytes, passthrough_threshold,
                    _flags(shared_tables, top_last), [b.data_ptr() for b in blobs], caps,
                    sizes.data_ptr(), ws.data_ptr(), ws.numel(), checksum_chunk_bytes,
                    [c.data_ptr() for c in crcs], ccaps)
    host_sizes = sizes.cpu().tolist()
    return ([b[:s] for b, s in zip(blobs, host_sizes)],
            [c[:(s + checksum_chunk_bytes - 1) // checksum_chunk_bytes] for c, s in zip(crcs, host_sizes)])


def compress_with_crc32(t, chunk_bytes=DEFAULT_CHUNK_BYTES, passthrough_threshold=DEFAULT_THRESHOLD,
                        checksum_chunk_bytes=DEFAULT_CRC_CHUNK_BYTES, shared_tables=False,
                        top_last=False):
    """(blob, checksums) of one GPU tensor (cuZipNN's compress_tensor_with_crc32)."""
    blobs, crcs = compress_batch_with_crc32([t], chunk_bytes, passthrough_threshold,
                                            checksum_chunk_bytes, shared_tables, top_last)
    return blobs[0], crcs[0]


def compress(t, chunk_bytes=DEFAULT_CHUNK_BYTES, passthrough_threshold=DEFAULT_THRESHOLD,
             shared_tables=False, top_last=False):
    """Blob (1-D uint8 tensor on t's device) of a GPU tensor's bytes."""
    return compress_batch([t], chunk_bytes, passthrough_threshold, shared_tables, top_last)[0]


def blob_info(blob_or_header):
    """Header fields as a dict; accepts a blob tensor (any device) or bytes."""
    hdr = _header_bytes(blob_or_header)
    info = Info()
    _check(lib().ltc_blob_info(hdr, len(hdr), ctypes.byref(info)), "blob_info")
    return {f: getattr(info, f) for f, _ in Info._fields_}


def _header_bytes(b):
    if isinstance(b, (bytes, bytearray)):
        return bytes(b[:64])
    return bytes(b[:64].cpu().numpy().tobytes())


def decompress_batch(blobs, shapes=None, check=True):
    """Decoded tensors (on the blobs' device) for up to 32 blobs."""
    if not 1 <= len(blobs) <= BATCH_MAX:
        raise ValueError(f"1..{BATCH_MAX} blobs per batch")
    headers = [_header_bytes(b) for b in blobs]
    infos = [blob_info(h) for h in headers]
    dev = blobs[0].device
    outs = [torch.empty(i["nbytes"], dtype=torch.uint8, device=dev) for i in infos]
    status = torch.full((len(blobs),), -99, dtype=torch.int32, device=dev)
    decompress_raw(headers, [b.data_ptr() for b in blobs], [b.numel() for b in blobs],
                   [o.data_ptr() for o in outs], [o.numel() for o in outs], status.data_ptr())
    if check:
        st = status.cpu().tolist()
        for s in st:
            _check(s, "decompress (device status)")
    res = []
    for k, (o, i) in enumerate(zip(outs, infos)):
        t = o.view(CODE_DTYPE[i["dtype"]])
        if shapes is not None and shapes[k] is not None:
            t = t.view(shapes[k])
        res.append(t)
    return res


def decompress(blob, shape=None):
    return decompress_batch([blob], [shape])[0]


def delta_workspace_size(headers):
    """Device workspace bytes for decoding these delta blobs (host headers)."""
    hdr = (ctypes.c_void_p * len(headers))(*[ctypes.cast(ctypes.c_char_p(h), ctypes.c_void_p)
                                             for h in headers])
    out = ctypes.c_uint64(0)
    _check(lib().ltc_decompress_delta_workspace_size(len(headers), hdr, ctypes.byref(out)),
           "delta workspace size")
    return out.value


def decompress_delta_raw(headers, blob_ptrs, blob_nbytes, base_ptrs, dst_ptrs, caps, status_ptr,
                         ws_ptr, ws_nbytes, stream=None):
    """Pointer-level batch decode of delta blobs on `stream`."""
    count = len(blob_ptrs)
    hdr = (ctypes.c_void_p * count)(*[ctypes.cast(ctypes.c_char_p(h), ctypes.c_void_p) for h in headers])
    _check(lib().ltc_decompress_delta_batch(count, hdr, _ptrs(blob_ptrs), _u64s(blob_nbytes),
                                            _ptrs(base_ptrs), _ptrs(dst_ptrs), _u64s(caps),
                                            ctypes.c_void_p(status_ptr), ctypes.c_void_p(ws_ptr),
                                            ws_nbytes, _stream(stream)), "decompress_delta")


def decompress_batch_delta(blobs, bases, shapes=None, check=True):
    """Tensors rebuilt from delta blobs and their bases (GPU tensors)."""
    if not 1 <= len(blobs) <= BATCH_MAX or len(bases) != len(blobs):
        raise ValueError(f"1..{BATCH_MAX} blobs per batch, one base each")
    headers = [_header_bytes(b) for b in blobs]
    infos = [blob_info(h) for h in headers]
    dev = blobs[0].device
    bs = [b.contiguous() for b in bases]
    for b, i in zip(bs, infos):
        if not b.is_cuda or b.numel() * b.element_size() != i["nbytes"]:
            raise ValueError("a base must be a GPU tensor of the blob's decoded size")
    outs = [torch.empty(i["nbytes"], dtype=torch.uint8, device=dev) for i in infos]
    ws_n = delta_workspace_size(headers)
    ws = torch.empty(max(ws_n, 256), dtype=torch.uint8, device=dev)
    status = torch.full((len(blobs),), -99, dtype=torch.int32, device=dev)
    decompress_delta_raw(headers, [b.data_ptr() for b in blobs], [b.numel() for b in blobs],
                         [b.data_ptr() for b in bs], [o.data_ptr() for o in outs],
                         [o.numel() for o in outs], status.data_ptr(), ws.data_ptr(), ws.numel())
    if check:
        for s in status.cpu().tolist():
            _check(s, "decompress_delta (device status)")
    res = []
    for k, (o, i) in enumerate(zip(outs, infos)):
        t = o.view(CODE_DTYPE[i["dtype"]])
        if shapes is not None and shapes[k] is not None:
            t = t.view(shapes[k])
        res.append(t)
    return res


def decompress_delta(blob, base, shape=None):
    """The tensor a delta blob codes, given its base."""
    return decompress_batch_delta([blob], [base], [shape])[0]


def decompress_from_host_raw(h_blob_ptrs, blob_nbytes, dst_ptrs, caps, status_ptr, stage_ptrs,
                             stage_caps, stream=None):
    """Pointer-level batch decode of blobs in host memory through device
    staging buffers, on `stream` (no allocation, no sync)."""
    count = len(h_blob_ptrs)
    _check(lib().ltc_decompress_batch_from_host(count, _ptrs(h_blob_ptrs), _u64s(blob_nbytes),
                                                _ptrs(dst_ptrs), _u64s(caps),
                                                ctypes.c_void_p(status_ptr), _ptrs(stage_ptrs),
                                                _u64s(stage_caps), _stream(stream)),
           "decompress_from_host")


def decompress_batch_from_host(blobs, shapes=None, device=None, check=True):
    """Decoded GPU tensors of up to 32 blobs held in CPU memory (uint8 CPU
    tensors, pinned for the copies to overlap the decoding)."""
    if not 1 <= len(blobs) <= BATCH_MAX:
        raise ValueError(f"1..{BATCH_MAX} blobs per batch")
    if any(b.is_cuda or b.dtype != torch.uint8 or not b.is_contiguous() for b in blobs):
        raise ValueError("blobs must be contiguous uint8 CPU tensors")
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    infos = [blob_info(_header_bytes(b)) for b in blobs]
    outs = [torch.empty(i["nbytes"], dtype=torch.uint8, device=dev) for i in infos]
    stages = [torch.empty(max(b.numel(), 16), dtype=torch.uint8, device=dev) for b in blobs]
    status = torch.full((len(blobs),), -99, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        decompress_from_host_raw([b.data_ptr() for b in blobs], [b.numel() for b in blobs],
                                 [o.data_ptr() for o in outs], [o.numel() for o in outs],
                                 status.data_ptr(), [st.data_ptr() for st in stages],
                                 [st.numel() for st in stages])
        st = status.cpu().tolist()  # synchronises: the host blobs are free again
    if check:
        for v in st:
            _check(v, "decompress_from_host (device status)")
    res = []
    for k, (o, i) in enumerate(zip(outs, infos)):
        t = o.view(CODE_DTYPE[i["dtype"]])
        if shapes is not None and shapes[k] is not None:
            t = t.view(shapes[k])
        res.append(t)
    return res


def decompress_from_host(blob, shape=None, device=None):
    """cuZipNN's decompress_tensor for a CPU blob: decoded on the GPU."""
    return decompress_batch_from_host([blob], [shape], device)[0]


def compress_to_host(t, chunk_bytes=DEFAULT_CHUNK_BYTES, passthrough_threshold=DEFAULT_THRESHOLD,
                     pin_memory=True, shared_tables=False, top_last=False):
    """cuZipNN's compress_tensor: the blob of a GPU tensor as a 1-D uint8 CPU
    tensor (pinned by default, ready for decompress_from_host)."""
    blob = compress(t, chunk_bytes, passthrough_threshold, shared_tables, top_last)
    out = torch.empty(blob.numel(), dtype=torch.uint8, pin_memory=pin_memory)
    out.copy_(blob)
    return out


def crc32_chunks(t, chunk_bytes=DEFAULT_CRC_CHUNK_BYTES):
    """CRC-32 (zlib's) of every chunk_bytes bytes of a GPU tensor, as int32 bits."""
    if not t.is_cuda:
        raise ValueError("tensor must be on a GPU")
    t = t.contiguous()
    nbytes = t.numel() * t.element_size()
    count = (nbytes + chunk_bytes - 1) // chunk_bytes if chunk_bytes else 0
    out = torch.empty(max(count, 1), dtype=torch.int32, device=t.device)
    _check(lib().ltc_crc32_chunks(ctypes.c_void_p(t.data_ptr()), nbytes, chunk_bytes,
                                  ctypes.c_void_p(out.data_ptr()), _stream()), "crc32_chunks")
    return out[:count]


def crc32_raw(src_ptrs, nbytes, chunk_bytes, crc_ptrs, stream=None, prepare=False):
    """Pointer-level batch CRC-32 on `stream` (no allocation, no sync).
    prepare: return a Prepared call instead of calling."""
    args = (len(src_ptrs), _ptrs(src_ptrs), _u64s(nbytes), chunk_bytes, _ptrs(crc_ptrs), _stream(stream))
    return _run(lib().ltc_crc32_chunks_batch, args, "crc32_chunks_batch", prepare)


def crc32_chunks_batch(tensors, chunk_bytes=DEFAULT_CRC_CHUNK_BYTES):
    """crc32_chunks for up to 32 GPU tensors in one launch."""
    ts = [t.contiguous() for t in tensors]
    if not 1 <= len(ts) <= BATCH_MAX or any(not t.is_cuda for t in ts):
        raise ValueError(f"1..{BATCH_MAX} GPU tensors per batch")
    nbytes = [t.numel() * t.element_size() for t in ts]
    counts = [(n + chunk_bytes - 1) // chunk_bytes if chunk_bytes else 0 for n in nbytes]
    outs = [torch.empty(max(c, 1), dtype=torch.int32, device=ts[0].device) for c in counts]
    crc32_raw([t.data_ptr() for t in ts], nbytes, chunk_bytes, [o.data_ptr() for o in outs])
    return [o[:c] for o, c in zip(outs, counts)]


def blob_stats(blob):
    """Mode counts and payload bytes per stream index (ZipNN Table II layout)."""
    info = blob_info(blob)
    prefix = bytes(blob[:info["payload_base"]].cpu().numpy().tobytes())
    st = Stats()
    _check(lib().ltc_blob_stats(prefix, len(prefix), ctypes.byref(st)), "blob_stats")
    e = st.elem_bytes
    return {
        "nbytes": st.nbytes, "blob_nbytes": st.blob_nbytes,
        "ratio": st.blob_nbytes / st.nbytes if st.nbytes else 0.0,
        "modes": [{"raw": st.mode_count[k][0], "rans": st.mode_count[k][1],
                   "const": st.mode_count[k][2], "zrun": st.mode_count[k][3]} for k in range(e)],
        "group_percent": [100.0 * st.payload_bytes[k] / st.stream_bytes[k]
                          if st.stream_bytes[k] else 0.0 for k in range(e)],
    }
