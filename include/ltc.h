/*
 * ltc.h -- C ABI of the MI355X (gfx950) lossless tensor codec.
 *
 * The library compresses the bytes of a tensor of model weights the way
 * ZipNN does ("NOTE-241: ZipNN" (nucleation notes), section "Method",
 * items 1-3 and 5): each element's bits are reordered so that the exponent
 * fills the top byte, the bytes are split into one stream per byte position
 * inside fixed-size chunks, and every stream is stored CONST (one repeated
 * value), RAW, or entropy coded with 64-lane interleaved rANS over a 256-bin
 * order-0 model normalised to a 4096 total.  The arguments and defaults
 * follow cuZipNN 0.1.0 (PyPI page, section "API": chunk_bytes = 131072, a
 * multiple of 8 and at most 16 MiB; passthrough_threshold = 0.95 in (0, 1];
 * CRC-32 per 16 KiB matching zlib.crc32, the last chunk shorter); the blob is
 * versioned and other versions are rejected (same page, "Blob format").  The
 * device-pointer, caller-stream, no-allocation convention follows lmz's
 * device entry point (lmz README, section "Building on lmz": the device
 * stays the caller's).
 *
 * OWNERSHIP AND ASYNCHRONY.  Arguments named d_* are device pointers, h_*
 * host pointers.  The caller allocates every buffer and owns the stream.
 * The library allocates no device memory, creates no context and never
 * synchronises: work is enqueued on `stream` and the call returns at once.
 * Results that only the device knows (*d_blob_nbytes, *d_status) are written
 * to device memory; read them after synchronising the stream.  Argument
 * errors the host can see are returned before anything is enqueued.  A HIP
 * launch failure returns LTC_ERR_HIP.  Calls on different streams are
 * independent.
 *
 * PIPELINED COMPRESSION.  A compress call over 4096 chunks or more (all
 * tensors of a batch together) in directory order, or of deltas, splits its
 * chunks into two chunk-ordered groups (a top-last call of that size runs on
 * `stream` alone: its encoder writes the top streams' payloads in place): the first runs on `stream`, the second on an internal
 * stream that waits for `stream` at the call and that `stream` waits for
 * before anything enqueued after the call, so the call still behaves as work
 * on `stream`.  One group's compute-bound encoding then overlaps another's
 * memory-bound passes.  The groups' offset scans run in chunk order, so blobs
 * are the same as from one group (in the top-last layout the top streams'
 * scans start after every group's lower-stream scan).  A caller that owns every stream (or
 * captures the call into a graph) passes LTC_FLAG_CALLER_STREAM_ONLY to
 * ltc_compress_batch_ex, and every kernel of the call then runs on `stream`
 * alone (measured on 28 BF16 tensors, 1.74 GB: 1.60 ms on one stream against
 * 1.44 ms in two groups).  Decoding blobs held in host memory
 * (ltc_decompress_from_host) likewise copies them on an internal stream
 * forked from and joined to `stream`.  The internal streams (default
 * priority) and events are the library's only state: created once per device
 * on first use, kept until the process ends, and used under a lock while a
 * call enqueues.  For compression, a stream of another device than the
 * current one, or the *_prof variants, run all chunks on `stream` alone; the
 * host-blob decode needs the stream to belong to the current device.
 *
 * BLOB FORMAT v1 (byte exact; all integers little-endian).
 *   dtype codes: LTC_U8 (element 1 byte), LTC_BF16, LTC_FP16 (2 bytes),
 *   LTC_FP32 (4 bytes).  E = element bytes, C = chunk_bytes, N = input bytes,
 *   K = ceil(N / C) chunks, S = K*E streams.
 *   Reorder: for BF16/FP16/FP32 (mantissa bits w_m = 7/10/23, W = 8E) the
 *   element x becomes y = e << (w_m+1) | s << w_m | m, i.e. the exponent
 *   field moves to the top and the sign sits just below it (for BF16 and
 *   FP32 the top byte is exactly the biased exponent).  U8 is not reordered.
 *   Stream k of chunk c holds byte k of y for every element of the chunk.
 *   Header, 64 bytes:
 *     0 'L','T','C','B' | 4 u16 version = 1 | 6 u8 dtype | 7 u8 E |
 *     8 u64 N | 16 u32 C | 20 u32 K | 24 u16 lanes = 64 | 26 u8 prob_bits
 *     = 12 | 27 u8 flags = 0 | 28 u32 0 | 32 u64 blob_nbytes |
 *     40 u64 payload_base = 64 + 16*S | 48 16 zero bytes
 *   Directory: S entries of 16 bytes, entry c*E + k:
 *     0 u64 offset from blob start | 8 u32 payload bytes | 12 u8 mode
 *     (0 RAW, 1 RANS, 2 CONST) | 13 u8 const value (0 unless CONST) | 14 u16 0
 *   Payloads in directory order, each at a multiple of 16: cursor starts at
 *   payload_base; offset = cursor; cursor = align16(cursor + size); the
 *   final cursor is blob_nbytes; every gap byte is zero.
 *   Mode choice for a stream of n bytes with histogram h: CONST if one value
 *   occurs; else the rANS payload size P is computed and the stream is RANS
 *   if P <= P_max(n), the largest integer strictly below
 *   passthrough_threshold * n in IEEE double, otherwise RAW (the n bytes).
 *   Frequencies: f[v] = 0 if h[v] = 0, else max(1, floor(h[v]*4096/n));
 *   while sum f > 4096, decrement the largest f > 1 (ties: smallest v); if
 *   sum f < 4096, add the shortfall to the largest h (ties: smallest v).
 *   rANS: 32-bit states, lower bound 2^16, 16-bit words, 64 lanes; symbol t
 *   belongs to lane t mod 64, step t / 64.  Encoding starts each lane at
 *   65536 and runs steps last to first, lanes 63 to 0: if x >= f[s] << 20,
 *   emit x & 0xFFFF and x >>= 16; then x = (x/f)*4096 + x%f + cum[s].
 *   Words are stored in decoding order: step by step, lanes ascending.
 *   RANS payload: 0 u32 W | 4 u8 sym_lo | 5 u8 sym_hi | 6 ten zero bytes |
 *     16 u32 states[64] | 272 u16 f[sym_lo..sym_hi] | zero pad to
 *     WO = align16(272 + 2*(sym_hi - sym_lo + 1)) | WO u16 words[W];
 *     payload bytes = WO + 2W.
 *   Decoding reverses this; a RANS stream must consume exactly W words and
 *   end with every state at 65536.
 *
 * BLOB FORMAT v2, SHARED TABLES (flag LTC_FLAG_SHARED_TABLES; lmz README,
 * "One format choice worth knowing about": one frequency table per plane
 * kind instead of one per rANS stream -- here a plane is a stream index k of
 * one blob, and sharing is the caller's choice):
 *   Header as v1 with version = 2 and flags (byte 27) = 1.
 *   After the directory, E table records, k = 0..E-1: 0 u16 lo | 2 u16 hi |
 *     4 twelve zero bytes | 16 u16 f[lo..hi] | zero pad to a multiple of 16;
 *     a plane with at most one distinct value in the whole blob has no table
 *     (lo = 1, hi = 0, 16 bytes).  payload_base = end of the records.
 *   Plane k's table: the v1 normalisation of the sum over all chunks of
 *     stream k's histograms.  A stream with one value is CONST; otherwise it
 *     is coded with its plane's table, payload 0 u32 W | 4 twelve zero bytes
 *     | 16 u32 states[64] | 272 u16 words[W] (272 + 2W bytes), RANS if that
 *     is at most P_max(n), else RAW.  Offsets and gaps as v1.
 *
 * DELTAS (header flag LTC_FLAG_DELTA, in v1 or v2; "NOTE-241: ZipNN",
 * section "Method" item 6 and the delta results: the XOR of two versions of
 * a model's weights, coded with a run coder instead of the order-0 coder
 * when a byte group is mostly zero bytes):
 *   The coded input is d = src XOR base, byte for byte; the header, reorder,
 *   streams and v1/v2 tables are those of the plain blob of d.  Directory
 *   mode 3 (ZRUN) adds a zero-run payload for a stream of n bytes:
 *     0 u32 nnz | 4 u32 nblk | 8 eight zero bytes | 16 bitmap of the
 *     ceil(n/64) 64-byte blocks, bit b (LSB first) set when block b holds a
 *     nonzero byte, zero pad to a multiple of 16 | nblk u64 masks, one per
 *     set block in order, bit j set when byte j of the block is nonzero,
 *     zero pad to a multiple of 16 | nnz nonzero bytes in stream order.
 *   Choice per stream: CONST if one value occurs; otherwise ZRUN is a
 *   candidate when 10*zeros > 9n or 100*(longest zero run) > 3n, and the
 *   smaller of the RANS and ZRUN payloads that are at most P_max(n) is
 *   stored (RANS on a tie); RAW if neither fits.  Decoding a delta blob
 *   needs the same base; without it, or with a base for a plain blob, the
 *   call returns INVALID_ARGUMENT.
 *
 * TOP-LAST LAYOUT (header flag LTC_FLAG_TOP_LAST, with v1, v2 and deltas;
 * "NOTE-241: ZipNN", section "Method" item 5: a map of the variable-size
 * compressed pieces lets each be found on its own -- here the directory,
 * whose offsets leave the order of the payloads free):
 *   Everything as without the flag except the order in which the cursor
 *   places payloads: first every stream k < E-1 in directory order (chunk
 *   by chunk), then every stream k = E-1 in chunk order.  Sizes, modes,
 *   payload bytes, gaps and blob_nbytes do not change; for E = 1 the two
 *   orders coincide.  The point is the compressor's memory traffic: the
 *   lower streams (for BF16 and FP32 mostly RAW sign/mantissa bytes, sized
 *   by the histogram pass) get their offsets before the top streams are
 *   coded, so the wave that codes a chunk's top stream, which loads every
 *   byte of its elements anyway, writes them straight into the blob.
 */
#ifndef LTC_H
#define LTC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LTC_U8 = 0, LTC_BF16 = 1, LTC_FP16 = 2, LTC_FP32 = 3 };

enum {
  LTC_OK = 0,
  LTC_ERR_INVALID_ARGUMENT = -1, /* bad size, chunk_bytes, threshold, pointer */
  LTC_ERR_UNSUPPORTED_DTYPE = -2,
  LTC_ERR_BAD_MAGIC = -3,
  LTC_ERR_BAD_VERSION = -4,      /* cuZipNN "Blob format": other versions rejected */
  LTC_ERR_CORRUPT = -5,          /* structural check failed */
  LTC_ERR_CAPACITY = -6,         /* output buffer too small */
  LTC_ERR_WORKSPACE = -7,        /* workspace too small */
  LTC_ERR_HIP = -8               /* a HIP call or launch failed */
};

enum { LTC_MODE_RAW = 0, LTC_MODE_RANS = 1, LTC_MODE_CONST = 2, LTC_MODE_ZRUN = 3 /* deltas */ };

#define LTC_FLAG_SHARED_TABLES 1u      /* compress flags: format v2 */
#define LTC_FLAG_DELTA 2u              /* header flag: XOR delta against a base */
#define LTC_FLAG_CALLER_STREAM_ONLY 4u /* compress flags: no internal stream, all on `stream` */
#define LTC_FLAG_TOP_LAST 8u           /* compress flags and header flag: top-last layout */
#define LTC_FLAG_PLACE_NO_WAIT 16u     /* compress flags, top-last: the encoder waits for no earlier
                                          payload size (see ltc_compress_batch_ex) */

#define LTC_HEADER_BYTES 64
#define LTC_DEFAULT_CHUNK_BYTES 131072u
#define LTC_DEFAULT_THRESHOLD 0.95
#define LTC_DEFAULT_CRC_CHUNK_BYTES 16384u
#define LTC_BATCH_MAX 32 /* tensors per batch call */

/* Parsed header (ltc_blob_info). */
typedef struct {
  int32_t dtype;
  uint32_t elem_bytes;
  uint64_t nbytes;       /* N: decoded size */
  uint32_t chunk_bytes;  /* C */
  uint32_t nchunks;      /* K */
  uint64_t blob_nbytes;
  uint64_t payload_base;
  uint32_t version;      /* 1, or 2 (shared tables) */
  uint32_t flags;        /* header byte 27: LTC_FLAG_SHARED_TABLES | LTC_FLAG_DELTA |
                            LTC_FLAG_TOP_LAST */
} ltc_info;

/* Element size of a dtype code, 0 if unknown. */
uint32_t ltc_elem_bytes(int dtype);

/* Upper bound of the blob size for an input of `nbytes` bytes:
 * 64 + 16*S + sum over streams of align16(stream bytes).  0 on bad args. */
uint64_t ltc_compress_bound(uint64_t nbytes, int dtype, uint32_t chunk_bytes);

/* Device workspace (bytes) that ltc_compress needs for this input. */
int ltc_compress_workspace_size(uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                                uint64_t* ws_nbytes);

/* Compress `nbytes` bytes at d_src (read as `dtype`, row-major) into d_blob.
 * d_src must be aligned to the element size; blob_capacity must be at least
 * ltc_compress_bound(); d_ws/ws_nbytes at least ltc_compress_workspace_size().
 * The blob size is written to *d_blob_nbytes (device u64).  The blob is
 * identical byte for byte to the format above for the same arguments.
 * Errors: INVALID_ARGUMENT (nbytes % E, chunk_bytes not a multiple of 8 or
 * outside [8, 2^24], threshold outside (0, 1], NULL pointers, K >= 2^32),
 * UNSUPPORTED_DTYPE, CAPACITY, WORKSPACE, HIP. */
int ltc_compress(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                 double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                 uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                 hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * blob as ltc_compress, with the workspace taken from a device array the
 * library holds on each GPU it runs on (LTC_NOALLOC_SCRATCH_BYTES = 64 MiB,
 * kept until the process ends; its address is looked up once per device, on
 * the first call there).  The call allocates nothing and uses no internal
 * stream: every kernel runs on `stream`, which must belong to the current
 * device.  The input is limited to what that workspace covers,
 * ltc_compress_workspace_size() <= LTC_NOALLOC_SCRATCH_BYTES (about 60 MB of
 * BF16 at the default chunk size); larger inputs return LTC_ERR_WORKSPACE
 * before anything is enqueued.  All calls on one GPU share its array: calls
 * whose work overlaps on that GPU (on different streams, or from several
 * threads) race and give undefined blobs; calls in order on one stream are
 * safe, since every call writes each workspace field it reads.  Other errors
 * as ltc_compress, plus INVALID_ARGUMENT for a stream of another device. */
#define LTC_NOALLOC_SCRATCH_BYTES (64ull << 20)
int ltc_compress_noalloc(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                         double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                         uint64_t* d_blob_nbytes, hipStream_t stream);

/* Batch of `count` (1..LTC_BATCH_MAX) tensors of one dtype, one launch
 * sequence; each blob is identical to what ltc_compress gives for that
 * tensor alone.  Host arrays hold the per-tensor device pointers and sizes;
 * d_blob_nbytes is a device array of `count` u64.  The workspace is
 * ltc_compress_batch_workspace_size(). */
int ltc_compress_batch_workspace_size(int count, const uint64_t* h_nbytes, int dtype,
                                      uint32_t chunk_bytes, uint64_t* ws_nbytes);
int ltc_compress_batch(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                       int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                       void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                       uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                       hipStream_t stream);

/* Parse and check the 64-byte header (a host copy of the blob's first bytes).
 * Errors: BAD_MAGIC, BAD_VERSION (cuZipNN "Blob format": blobs of other
 * versions are rejected), UNSUPPORTED_DTYPE, CORRUPT (inconsistent fields). */
int ltc_blob_info(const void* h_header, uint64_t h_nbytes, ltc_info* out);

/* Decode a blob into d_dst (dst_capacity >= N).  h_header is a host copy of
 * the blob's first 64 bytes (the host needs N, C and K to size the launch);
 * blob_nbytes must equal the header's blob_nbytes.  The kernels validate the
 * directory and every payload against the format (offset chain, sizes,
 * modes, table sums, states, word counts, end states) without ever reading
 * or writing out of bounds, and write LTC_OK or LTC_ERR_CORRUPT to *d_status
 * (device i32).  After CORRUPT the contents of d_dst are unspecified.  A
 * checksum is still the way to detect a corrupted payload that happens to
 * decode (cuZipNN "API": verify untrusted blobs with CRC-32 first).  A delta
 * blob (LTC_FLAG_DELTA) is refused with INVALID_ARGUMENT here and in the
 * other base-less decode calls: ltc_decompress_delta decodes it. */
int ltc_decompress(const void* h_header, const void* d_blob, uint64_t blob_nbytes,
                   void* d_dst, uint64_t dst_capacity, int32_t* d_status,
                   hipStream_t stream);

/* Batch decode of `count` (1..LTC_BATCH_MAX) blobs of one dtype and chunk
 * size; d_status is a device array of `count` i32. */
int ltc_decompress_batch(int count, const void* const* h_headers,
                         const void* const* h_blob_ptrs, const uint64_t* h_blob_nbytes,
                         void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                         int32_t* d_status, hipStream_t stream);

/* Decode a blob held in host memory (cuZipNN 0.1.0 "API": decompress_tensor
 * takes a blob on the CPU and decodes on the GPU; lmz README, "On a GPU":
 * once decoding outruns the host link, the ratio becomes load bandwidth).
 * h_blob is the whole blob (blob_nbytes bytes) in host memory, pinned
 * (hipHostMalloc) for the copies to overlap; d_stage is a device buffer of
 * stage_capacity >= blob_nbytes bytes, 16-byte aligned, that receives it.
 * The blob is copied in chunk-ordered groups on a library-internal stream
 * (forked from and joined to `stream`), and each group is decoded on
 * `stream` as soon as its bytes have arrived.  The host reads the header and
 * the directory from h_blob to size the copies; h_blob must stay unchanged
 * until the call's work on `stream` has finished.  Output, status and errors
 * as ltc_decompress, plus CAPACITY for a short staging buffer. */
int ltc_decompress_from_host(const void* h_blob, uint64_t blob_nbytes, void* d_dst,
                             uint64_t dst_capacity, int32_t* d_status, void* d_stage,
                             uint64_t stage_capacity, hipStream_t stream);

/* Batch form: `count` (1..LTC_BATCH_MAX) host blobs of one dtype and chunk
 * size, each with its own staging buffer; d_status holds `count` i32. */
int ltc_decompress_batch_from_host(int count, const void* const* h_blobs, const uint64_t* h_blob_nbytes,
                                   void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                                   int32_t* d_status, void* const* h_stage_ptrs,
                                   const uint64_t* h_stage_capacity, hipStream_t stream);

/* CRC-32 (zlib's: reflected 0xEDB88320, init and final xor 0xFFFFFFFF) of
 * every chunk_bytes-byte chunk of d_src, the last one possibly shorter
 * (cuZipNN 0.1.0 "API", hash_tensor_with_crc32).  d_crc receives
 * ceil(nbytes / chunk_bytes) u32 values.  chunk_bytes >= 1. */
int ltc_crc32_chunks(const void* d_src, uint64_t nbytes, uint32_t chunk_bytes,
                     uint32_t* d_crc, hipStream_t stream);

/* The same for `count` (1..LTC_BATCH_MAX) buffers in one launch; buffer i's
 * checksums go to h_crc_ptrs[i] (a device pointer held in a host array). */
int ltc_crc32_chunks_batch(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                           uint32_t chunk_bytes, uint32_t* const* h_crc_ptrs, hipStream_t stream);

/* Upper bound of the blob size with compress flags (0: ltc_compress_bound;
 * LTC_FLAG_SHARED_TABLES adds E table records of at most 528 bytes;
 * LTC_FLAG_CALLER_STREAM_ONLY, LTC_FLAG_TOP_LAST and LTC_FLAG_PLACE_NO_WAIT
 * change nothing).  0 on bad arguments. */
uint64_t ltc_compress_bound_ex(uint64_t nbytes, int dtype, uint32_t chunk_bytes, uint32_t flags);

/* The general compress call: ltc_compress_batch plus
 *   flags: 0 (format v1) or LTC_FLAG_SHARED_TABLES (format v2), either with
 *     LTC_FLAG_TOP_LAST (the top-last layout); capacities are checked
 *     against ltc_compress_bound_ex; with LTC_FLAG_CALLER_STREAM_ONLY added,
 *     the call uses no internal stream (same blobs, all kernels on `stream`
 *     one after another); with LTC_FLAG_PLACE_NO_WAIT added to a top-last
 *     call, the encoder waves that place top-stream payloads (calls of 4096
 *     chunks or more, no deltas) wait for no earlier payload's size: a wave
 *     whose offset is not known the moment it looks leaves its payload to
 *     the packing pass, the fallback a slow predecessor otherwise triggers.
 *     Same blobs; for testing that path;
 *   h_base_ptrs: NULL, or per tensor the device pointer of its delta base
 *     (nbytes bytes, aligned like the source): the blobs are XOR deltas
 *     (LTC_FLAG_DELTA set in the header; with checksums the CRC kernel reads
 *     the finished blobs back);
 *   checksum_chunk_bytes: 0, or the CRC-32 of the blobs as in
 *     ltc_compress_batch_with_crc32 (h_crc_ptrs / h_crc_capacity);
 *   h_events: NULL, or the events of the *_prof variants (5, or 6 with
 *     checksums), and then every kernel runs on `stream` one after another.
 * v2 first builds every plane's table from the histograms of all chunks,
 * then codes the chunks (in groups on several streams, as v1). */
int ltc_compress_batch_ex(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                          int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                          uint32_t flags, const void* const* h_base_ptrs, void* const* h_blob_ptrs,
                          const uint64_t* h_blob_capacity, uint64_t* d_blob_nbytes,
                          uint32_t checksum_chunk_bytes, uint32_t* const* h_crc_ptrs,
                          const uint64_t* h_crc_capacity, void* d_ws, uint64_t ws_nbytes,
                          hipStream_t stream, const hipEvent_t* h_events);

/* XOR delta of d_src against d_base ("NOTE-241: ZipNN", "Method" item 6;
 * format above, DELTAS): both nbytes bytes of `dtype`, aligned to the
 * element size.  flags: 0, LTC_FLAG_SHARED_TABLES, LTC_FLAG_TOP_LAST, or
 * both.  Capacity, workspace
 * (ltc_compress_workspace_size) and errors as ltc_compress, plus
 * INVALID_ARGUMENT for a NULL or misaligned base. */
int ltc_compress_delta(const void* d_src, const void* d_base, uint64_t nbytes, int dtype,
                       uint32_t chunk_bytes, double passthrough_threshold, uint32_t flags, void* d_blob,
                       uint64_t blob_capacity, uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                       hipStream_t stream);

/* Device workspace for decoding these delta blobs: the sum over blobs of
 * K * E * align16(floor(C / E)) bytes (each stream gets a 16-byte aligned
 * slot its ZRUN payload is expanded into before the decode kernel reads it as
 * a RAW stream, 8 bytes at a time). */
int ltc_decompress_delta_workspace_size(int count, const void* const* h_headers, uint64_t* ws_nbytes);

/* Decode delta blobs: output = decoded delta XOR base.  h_base_ptrs[i] is a
 * device pointer to blob i's base (N bytes, aligned to the element size);
 * d_ws/ws_nbytes at least ltc_decompress_delta_workspace_size().  Every ZRUN
 * payload is checked (counts, block bitmap and masks agree, no zero
 * literal, exact size) before use.  Status and errors as
 * ltc_decompress_batch, plus INVALID_ARGUMENT for a plain blob, a NULL or
 * misaligned base, and WORKSPACE. */
int ltc_decompress_delta_batch(int count, const void* const* h_headers, const void* const* h_blob_ptrs,
                               const uint64_t* h_blob_nbytes, const void* const* h_base_ptrs,
                               void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                               int32_t* d_status, void* d_ws, uint64_t ws_nbytes, hipStream_t stream);
int ltc_decompress_delta(const void* h_header, const void* d_blob, uint64_t blob_nbytes,
                         const void* d_base, void* d_dst, uint64_t dst_capacity, int32_t* d_status,
                         void* d_ws, uint64_t ws_nbytes, hipStream_t stream);

/* Compress and checksum the blob in one call (cuZipNN 0.1.0 "API",
 * compress_tensor_with_crc32): the same blob as ltc_compress, and in d_crc
 * one CRC-32 per consecutive checksum_chunk_bytes bytes of the blob (a
 * shorter final piece included), exactly as ltc_crc32_chunks would give for
 * the finished blob.  The blob size is known only on the device, so d_crc must
 * hold crc_capacity >= ceil(ltc_compress_bound() / checksum_chunk_bytes)
 * u32 values; the first ceil(*d_blob_nbytes / checksum_chunk_bytes) are
 * written and the rest are left as they were.  When checksum_chunk_bytes is a
 * multiple of 1 KiB and at most 1 MiB, the payload is checksummed while it
 * is written (k_pack) and only the chunks holding header or directory bytes
 * and the blob's last chunk are read back; otherwise the CRC kernel reads
 * the blob back after packing.  The workspace is the same
 * as for ltc_compress.  Errors: those of ltc_compress, INVALID_ARGUMENT for
 * checksum_chunk_bytes = 0 or a NULL or misaligned d_crc, CAPACITY for a
 * short crc_capacity. */
int ltc_compress_with_crc32(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                            double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                            uint64_t* d_blob_nbytes, uint32_t checksum_chunk_bytes, uint32_t* d_crc,
                            uint64_t crc_capacity, void* d_ws, uint64_t ws_nbytes,
                            hipStream_t stream);

/* Batch form: tensor i's checksums go to h_crc_ptrs[i] (a device pointer in
 * a host array) with h_crc_capacity[i] entries; the workspace is
 * ltc_compress_batch_workspace_size(). */
int ltc_compress_batch_with_crc32(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                                  int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                                  void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                                  uint64_t* d_blob_nbytes, uint32_t checksum_chunk_bytes,
                                  uint32_t* const* h_crc_ptrs, const uint64_t* h_crc_capacity,
                                  void* d_ws, uint64_t ws_nbytes, hipStream_t stream);

/* Statistics from a host copy of the header and directory (the first
 * payload_base bytes): per stream-index mode counts and payload bytes (the
 * per-byte-group layout of ZipNN's Table II) and the whole-blob ratio. */
typedef struct {
  uint32_t elem_bytes;
  uint64_t nbytes;
  uint64_t blob_nbytes;
  uint64_t mode_count[4][4];     /* [stream index k][mode]; mode 3 only in deltas */
  uint64_t payload_bytes[4];     /* sum of payload sizes per stream index */
  uint64_t stream_bytes[4];      /* sum of raw stream sizes per stream index */
} ltc_stats;
int ltc_blob_stats(const void* h_prefix, uint64_t h_nbytes, ltc_stats* out);

/* Profiling variants: identical work and results, all on `stream` kernel by
 * kernel (never pipelined), plus hipEventRecord on `stream` around each kernel
 * so a caller can time one kernel alone.
 * Compress: 5 events (before k_hist, before k_encode, before k_scan, before
 * k_pack, after k_pack; in the top-last layout, format v1, the lower streams'
 * k_encode and scan come before the second event, so that the second
 * interval holds the top streams' k_encode alone); compress with CRC-32: 6,
 * the sixth after the CRC kernel that finishes the checksums.  Decompress: 3 events (before the
 * single-table decode kernel, between it and the multi-table one, after). */
int ltc_compress_batch_prof(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                            int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                            void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                            uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                            hipStream_t stream, const hipEvent_t* h_events);
int ltc_compress_batch_with_crc32_prof(int count, const void* const* h_src_ptrs,
                                       const uint64_t* h_nbytes, int dtype, uint32_t chunk_bytes,
                                       double passthrough_threshold, void* const* h_blob_ptrs,
                                       const uint64_t* h_blob_capacity, uint64_t* d_blob_nbytes,
                                       uint32_t checksum_chunk_bytes, uint32_t* const* h_crc_ptrs,
                                       const uint64_t* h_crc_capacity, void* d_ws,
                                       uint64_t ws_nbytes, hipStream_t stream,
                                       const hipEvent_t* h_events);
int ltc_decompress_batch_prof(int count, const void* const* h_headers,
                              const void* const* h_blob_ptrs, const uint64_t* h_blob_nbytes,
                              void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                              int32_t* d_status, hipStream_t stream, const hipEvent_t* h_events);

#ifdef __cplusplus
}
#endif
#endif
