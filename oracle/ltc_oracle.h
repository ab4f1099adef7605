/*
 * ltc_oracle.h -- plain, slow, scalar CPU oracle for the lossless tensor codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library may include,
 * link or call this file.  It is used by tests/, by __graft_entry__.smoke()
 * and by the cpu_baseline leg of bench.py, and by nothing else.  It shares no
 * source, header, table or helper with the HIP implementation; both are
 * written independently from the same format description (below).
 *
 * What it computes (pages cited by title and section):
 *  - ZipNN's method as summarised in "NOTE-241: ZipNN" (nucleation notes),
 *    section "Method", items 1-3 and 5: exponent extraction, byte grouping,
 *    order-0 entropy coding per stream, all-zero (here: single-valued)
 *    streams reduced to a header, independent fixed-size chunks with a map.
 *  - cuZipNN 0.1.0 (PyPI page), section "API": chunk_bytes (multiple of 8,
 *    at most 16 MiB), passthrough_threshold in (0, 1] (coding is kept only
 *    when it makes a stream smaller than that fraction of its size),
 *    per-chunk CRC-32 that matches zlib.crc32 with a shorter last chunk;
 *    section "Blob format": a versioned blob, other versions rejected.
 *  - lmz (lmzip 1.3.0 README), sections "On a GPU" and "Building on lmz":
 *    rANS with several interleaved states as lanes of work, and a frequency
 *    table carried per rANS stream.
 *
 * Format v1 (all integers little-endian).  Where the pages leave a step open
 * the plainest reading was taken; each reading is marked READING.
 *
 *  dtype codes: 0 U8 (E=1), 1 BF16 (E=2), 2 FP16 (E=2), 3 FP32 (E=4).
 *  Reorder (READING: "the exponent fills one byte"): for BF16/FP16/FP32 with
 *  W = 8E bits and w_m mantissa bits (7/10/23) the exponent field moves to
 *  the top bits, the sign sits directly below it, the mantissa is unchanged:
 *     y = e << (w_m+1) | s << w_m | m.     U8: y = x.
 *  Chunk c covers bytes [c*C, min((c+1)*C, N)); n_c = its element count.
 *  Stream k (k = 0..E-1) of chunk c = byte k of y for each element, in order.
 *  Per stream: h = 256-bin histogram.
 *    one distinct value      -> CONST (payload 0 bytes, value in directory)
 *    else normalise (below), rANS-encode -> payload size P;
 *    P <= P_max(n) -> RANS, else RAW (payload = the n stream bytes), where
 *    P_max(n) is the largest integer P with (double)P < theta*(double)n.
 *  Normalisation to M = 4096 (READING; the pages only fix the 2^12 total):
 *    f[v] = 0 if h[v] = 0 else max(1, floor(h[v]*4096/n));
 *    while sum f > 4096: decrement the largest f[v] > 1 (ties: smallest v);
 *    if sum f < 4096: add the shortfall to the v with the largest h[v]
 *    (ties: smallest v).
 *  rANS (READING of "interleaved-lane rANS"): 32-bit state, lower bound
 *    2^16, 16-bit renormalisation words, 64 lanes; symbol t is coded by lane
 *    t mod 64 at step t / 64.  The encoder starts every lane at 65536 and
 *    walks steps from last to first and lanes from 63 to 0; before coding s
 *    it emits the low 16 bits of x (and shifts x right by 16) when
 *    x >= f[s] << 20; then x = (x / f[s]) * 4096 + x % f[s] + cum[s].
 *    The word list is stored in decoder read order (reverse of emission).
 *  RANS payload: u32 W | u8 sym_lo | u8 sym_hi | 10 zero bytes |
 *    u32 states[64] | u16 f[sym_lo..sym_hi] | zero pad to WO = align16(272+2T)
 *    | u16 words[W];  P = WO + 2W, T = sym_hi - sym_lo + 1.
 *  Blob: 64-byte header, then S = K*E directory entries of 16 bytes, then
 *    payloads, each starting at a multiple of 16; gaps are zero.
 *    header: "LTCB" | u16 version=1 | u8 dtype | u8 E | u64 N | u32 C |
 *            u32 K | u16 lanes=64 | u8 prob_bits=12 | u8 flags=0 | u32 0 |
 *            u64 blob_nbytes | u64 payload_base=64+16S | 16 zero bytes
 *    entry:  u64 offset | u32 payload_nbytes | u8 mode (0 RAW,1 RANS,2 CONST)
 *            | u8 const value | u16 0
 *    offsets: cursor = payload_base; each entry in order gets offset =
 *    cursor, cursor = align16(cursor + size); blob_nbytes = final cursor.
 *  CRC-32: reflected polynomial 0xEDB88320, init and final xor 0xFFFFFFFF
 *    (the zlib / ISO-HDLC CRC), computed afresh per chunk.
 *
 * Format v2, shared tables (lmz README, "One format choice worth knowing
 * about": one frequency table per plane kind instead of one per rANS stream;
 * READING: a plane is a stream index k of one blob, and sharing is the
 * caller's choice, not decided per plane):
 *  header as v1 but version = 2 and flags (byte 27) = 1.
 *  After the directory come E table records, k = 0..E-1:
 *    u16 lo | u16 hi | 12 zero bytes | u16 f[lo..hi] | zero pad to 16;
 *    a plane without a table (at most one value over the whole blob):
 *    lo = 1, hi = 0, 16 bytes.
 *  payload_base = end of the records.  Table of plane k: normalise (as v1)
 *    the sum over all chunks of stream k's histograms.
 *  Per stream: one value -> CONST; else rANS with the plane's table, payload
 *    u32 W | 12 zero bytes | u32 states[64] | u16 words[W], P = 272 + 2W;
 *    P <= P_max(n) -> RANS, else RAW.  Offsets and gaps as v1.
 *
 * Deltas (NOTE-241: ZipNN, "Method" item 6; "Key results", Deltas): the
 * input is src XOR base, byte for byte, before everything above; header
 * flag bit 1 (value 2) marks a delta blob (flags 2 in v1, 3 in v2).  ZipNN
 * picks a run coder over its order-0 coder for a byte group when more than
 * 90% of it is zero bytes or a zero run exceeds 3% of it (READING: integers,
 * 10*zeros > 9n or 100*longest_zero_run > 3n, per chunk stream).  Here the
 * rule admits a ZRUN payload (mode 3) as a candidate; the stream takes the
 * smaller of RANS and ZRUN (ties: RANS), RAW if neither is <= P_max(n).
 *  ZRUN payload: u32 nnz | u32 nblk | 8 zero bytes | bitmap of the nonzero
 *    64-byte blocks (ceil(n/64) bits, LSB first), zero pad to 16 | nblk u64
 *    masks (bit i = byte i of the block is nonzero), zero pad to 16 | the
 *    nnz nonzero bytes in order.
 *
 * Top streams last (header flag bit 3, value 8; with v1, v2 and deltas):
 * NOTE-241: ZipNN, "Method" item 5 keeps a map of the variable-size
 * compressed pieces so each can be found on its own; the directory is that
 * map, which leaves the order of the payloads free (READING).  In this layout
 * the cursor first walks every stream k < E-1 in directory order, then every
 * stream k = E-1 (the exponent byte of BF16 and FP32, "Method" item 1) in
 * chunk order.  Entries, payloads, gaps and blob_nbytes are otherwise those
 * of the same blob without the flag; for E = 1 the two orders coincide.
 */
#ifndef LTC_ORACLE_H
#define LTC_ORACLE_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes (part of the format contract; same values as the library's) */
#define LTCO_OK 0
#define LTCO_ERR_INVALID_ARGUMENT (-1)
#define LTCO_ERR_UNSUPPORTED_DTYPE (-2)
#define LTCO_ERR_BAD_MAGIC (-3)
#define LTCO_ERR_BAD_VERSION (-4)
#define LTCO_ERR_CORRUPT (-5)
#define LTCO_ERR_CAPACITY (-6)

#define LTCO_FLAG_SHARED_TABLES 1u /* compress_ex: format v2 */
#define LTCO_FLAG_DELTA 2u         /* header flag: XOR delta against a base */
#define LTCO_FLAG_TOP_LAST 8u      /* payloads of stream E-1 after all others */

#define LTCO_MODE_RAW 0
#define LTCO_MODE_RANS 1
#define LTCO_MODE_CONST 2
#define LTCO_MODE_ZRUN 3 /* delta blobs only */

int ltco_elem_bytes(int dtype);
uint32_t ltco_reorder(int dtype, uint32_t x);
uint32_t ltco_unreorder(int dtype, uint32_t y);

/* bytes of stream k of chunk c (n_c bytes written to out); returns n_c */
uint64_t ltco_chunk_stream(const uint8_t* src, uint64_t nbytes, int dtype,
                           uint32_t chunk_bytes, uint64_t c, int k, uint8_t* out);
void ltco_histogram(const uint8_t* sym, uint64_t n, uint64_t h[256]);
int ltco_normalize(const uint64_t h[256], uint16_t f[256]);
uint64_t ltco_p_max(uint64_t n, double theta);
/* words_cap must be >= n; returns LTCO_OK or an error */
int ltco_rans_encode(const uint8_t* sym, uint64_t n, const uint16_t f[256],
                     uint32_t states[64], uint16_t* words, uint64_t words_cap,
                     uint64_t* nwords);
int ltco_rans_decode(const uint16_t* words, uint64_t nwords,
                     const uint32_t states[64], const uint16_t f[256],
                     uint64_t n, uint8_t* out);

uint64_t ltco_compress_bound(uint64_t nbytes, int dtype, uint32_t chunk_bytes);
int ltco_compress(const uint8_t* src, uint64_t nbytes, int dtype,
                  uint32_t chunk_bytes, double theta, uint8_t* blob,
                  uint64_t blob_capacity, uint64_t* blob_nbytes, int nthreads);
/* flags 0: ltco_compress (v1); LTCO_FLAG_SHARED_TABLES: format v2;
 * LTCO_FLAG_TOP_LAST (with either): top streams placed last */
uint64_t ltco_compress_bound_ex(uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                                uint32_t flags);
int ltco_compress_ex(const uint8_t* src, uint64_t nbytes, int dtype,
                     uint32_t chunk_bytes, double theta, uint32_t flags,
                     uint8_t* blob, uint64_t blob_capacity, uint64_t* blob_nbytes,
                     int nthreads);
/* the E payloads of one chunk, each zero-padded to a multiple of 16 and
 * concatenated; modes/cvals/sizes get one entry per stream; *nout = bytes */
int ltco_encode_chunk(const uint8_t* src, uint64_t nbytes, int dtype,
                      uint32_t chunk_bytes, double theta, uint64_t c,
                      uint8_t* modes, uint8_t* cvals, uint32_t* sizes,
                      uint8_t* out, uint64_t out_cap, uint64_t* nout);
int ltco_decompress(const uint8_t* blob, uint64_t blob_nbytes, uint8_t* dst,
                    uint64_t dst_capacity, uint64_t* out_nbytes, int nthreads);
/* deltas: compress src XOR base (flags: LTCO_FLAG_SHARED_TABLES, LTCO_FLAG_TOP_LAST); decode
 * and XOR the base back in.  A delta blob needs its base and only then. */
int ltco_compress_delta(const uint8_t* src, const uint8_t* base, uint64_t nbytes, int dtype,
                        uint32_t chunk_bytes, double theta, uint32_t flags, uint8_t* blob,
                        uint64_t blob_capacity, uint64_t* blob_nbytes, int nthreads);
int ltco_decompress_delta(const uint8_t* blob, uint64_t blob_nbytes, const uint8_t* base,
                          uint8_t* dst, uint64_t dst_capacity, uint64_t* out_nbytes,
                          int nthreads);

uint32_t ltco_crc32(const uint8_t* p, uint64_t n);
int ltco_crc32_chunks(const uint8_t* p, uint64_t n, uint32_t chunk_bytes,
                      uint32_t* out);

#ifdef __cplusplus
}
#endif
#endif
