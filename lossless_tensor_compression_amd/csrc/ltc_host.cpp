// ltc_host.cpp -- host-only code that reads blob bytes: the 64-byte header
// check (ltc_blob_info), directory statistics (ltc_blob_stats) and the copy
// groups of blobs held in host memory.  Plain C++ (no HIP): the library links
// it, and the CPU tests also build it with -fsanitize=address,undefined and
// feed it truncated and bit-flipped headers and directories.
//
// The header layout and its checks follow the blob format in include/ltc.h:
// a versioned blob whose other versions are rejected (cuZipNN 0.1.0, "Blob
// format"), and structural validation instead of undefined behaviour on a
// foreign blob (cuZipNN 0.1.0, "API", which leaves it undefined).
#include <string.h>

#include "ltc.h"
#include "ltc_format.h"
#include "ltc_host.h"

namespace ltc {
namespace {

uint64_t rd64(const uint8_t* p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}
uint32_t rd32(const uint8_t* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}
uint16_t rd16(const uint8_t* p) {
  uint16_t v;
  memcpy(&v, p, 2);
  return v;
}

// byte offset of stream s from its directory entry (the caller keeps s
// below the header's K*E)
uint64_t dir_offset(const uint8_t* blob, uint64_t s) { return rd64(blob + kHeader + kDirEntry * s); }

}  // namespace

uint32_t elem_bytes(int dtype) {
  switch (dtype) {
    case LTC_U8: return 1;
    case LTC_BF16: return 2;
    case LTC_FP16: return 2;
    case LTC_FP32: return 4;
    default: return 0;
  }
}

uint64_t host_copy_groups(uint64_t total_bytes, uint64_t total_chunks, uint64_t group_bytes,
                          uint64_t max_groups) {
  if (total_chunks == 0) return 0;
  uint64_t g = group_bytes ? total_bytes / group_bytes : 1;
  if (g < 1) g = 1;
  if (g > max_groups) g = max_groups;
  if (g > total_chunks) g = total_chunks;
  return g;
}

uint32_t host_group_ranges(const HostBlob* blobs, uint32_t count, uint32_t e, uint64_t T,
                           uint64_t G, uint64_t g, HostRange* out) {
  if (G == 0 || g >= G) return 0;
  const uint64_t c0 = T * g / G, c1 = T * (g + 1) / G;
  uint32_t n = 0;
  for (uint32_t j = 0; j < count; ++j) {
    const HostBlob& b = blobs[j];
    if (c1 <= b.chunk0 || c0 >= b.chunk0 + b.nchunks) continue;  // no chunk of blob j here
    const uint64_t lo_c = c0 > b.chunk0 ? c0 - b.chunk0 : 0;
    const uint64_t hi_c = c1 - b.chunk0 < b.nchunks ? c1 - b.chunk0 : b.nchunks;
    const uint64_t B = b.nbytes;
    auto put = [&](uint64_t lo, uint64_t hi) {
      lo = lo < B ? lo : B;
      hi = hi < lo ? lo : (hi < B ? hi : B);
      if (hi > lo) out[n++] = HostRange{j, lo, hi};
    };
    if (!b.top_last || e == 1) {
      put(lo_c == 0 ? 0 : dir_offset(b.data, lo_c * e), hi_c == b.nchunks ? B : dir_offset(b.data, hi_c * e));
    } else {
      // lower streams from stream 0 of the first chunk; top streams from
      // stream E-1 of the first chunk; each up to the same stream of the
      // next group's first chunk, or to where the part ends
      const uint64_t top0 = dir_offset(b.data, e - 1);  // the first top stream
      put(lo_c == 0 ? 0 : dir_offset(b.data, lo_c * e), hi_c == b.nchunks ? top0 : dir_offset(b.data, hi_c * e));
      put(dir_offset(b.data, lo_c * e + e - 1), hi_c == b.nchunks ? B : dir_offset(b.data, hi_c * e + e - 1));
    }
  }
  return n;
}

}  // namespace ltc

using ltc::elem_bytes;
using ltc::kDirEntry;
using ltc::kHeader;
using ltc::kLanes;
using ltc::kProbBits;

extern "C" {

uint32_t ltc_elem_bytes(int dtype) { return elem_bytes(dtype); }

int ltc_blob_info(const void* h_header, uint64_t h_nbytes, ltc_info* out) {
  if (!h_header || !out) return LTC_ERR_INVALID_ARGUMENT;
  if (h_nbytes < kHeader) return LTC_ERR_CORRUPT;
  const uint8_t* h = static_cast<const uint8_t*>(h_header);
  if (memcmp(h, "LTCB", 4) != 0) return LTC_ERR_BAD_MAGIC;
  const uint32_t version = ltc::rd16(h + 4);
  if (version != 1 && version != 2) return LTC_ERR_BAD_VERSION;
  const int dtype = h[6];
  const uint32_t e = elem_bytes(dtype);
  if (!e) return LTC_ERR_UNSUPPORTED_DTYPE;
  if (h[7] != e) return LTC_ERR_CORRUPT;
  const uint64_t nbytes = ltc::rd64(h + 8);
  const uint32_t chunk_bytes = ltc::rd32(h + 16);
  const uint64_t k = ltc::rd32(h + 20);
  if (ltc::rd16(h + 24) != kLanes || h[26] != kProbBits ||
      (h[27] & ~(LTC_FLAG_DELTA | LTC_FLAG_TOP_LAST)) != (version == 2 ? LTC_FLAG_SHARED_TABLES : 0u) ||
      ltc::rd32(h + 28) != 0)
    return LTC_ERR_CORRUPT;
  for (int i = 48; i < 64; ++i)
    if (h[i]) return LTC_ERR_CORRUPT;
  if (chunk_bytes < 8 || chunk_bytes > (1u << 24) || chunk_bytes % 8) return LTC_ERR_CORRUPT;
  if (nbytes % e) return LTC_ERR_CORRUPT;
  // K = ceil(N / C), computed without wrapping for any N
  if (k != nbytes / chunk_bytes + (nbytes % chunk_bytes != 0)) return LTC_ERR_CORRUPT;
  // v2: E table records of 16 to 528 bytes between the directory and the payloads
  const uint64_t dir_end = kHeader + kDirEntry * k * e;
  const uint64_t base = ltc::rd64(h + 40);
  const uint64_t blob_nbytes = ltc::rd64(h + 32);
  if (version == 1 ? base != dir_end
                   : (base < dir_end + 16ull * e || base > dir_end + 528ull * e || base % 16))
    return LTC_ERR_CORRUPT;
  if (blob_nbytes < base || blob_nbytes % 16) return LTC_ERR_CORRUPT;
  out->dtype = dtype;
  out->elem_bytes = e;
  out->nbytes = nbytes;
  out->chunk_bytes = chunk_bytes;
  out->nchunks = (uint32_t)k;
  out->blob_nbytes = blob_nbytes;
  out->payload_base = base;
  out->version = version;
  out->flags = h[27];
  return LTC_OK;
}

int ltc_blob_stats(const void* h_prefix, uint64_t h_nbytes, ltc_stats* out) {
  ltc_info info;
  const int rc = ltc_blob_info(h_prefix, h_nbytes, &info);
  if (rc) return rc;
  if (!out || h_nbytes < info.payload_base) return LTC_ERR_INVALID_ARGUMENT;
  memset(out, 0, sizeof(*out));
  out->elem_bytes = info.elem_bytes;
  out->nbytes = info.nbytes;
  out->blob_nbytes = info.blob_nbytes;
  const uint8_t* d = static_cast<const uint8_t*>(h_prefix) + kHeader;
  const uint32_t e = info.elem_bytes;
  const uint32_t max_mode = (static_cast<const uint8_t*>(h_prefix)[27] & LTC_FLAG_DELTA) ? 3u : 2u;
  for (uint64_t c = 0; c < info.nchunks; ++c) {
    const uint64_t len = c + 1 < info.nchunks ? info.chunk_bytes : info.nbytes - c * (uint64_t)info.chunk_bytes;
    for (uint32_t k = 0; k < e; ++k) {
      const uint8_t* ent = d + kDirEntry * (c * e + k);
      const uint32_t mode = ent[12];
      if (mode > max_mode) return LTC_ERR_CORRUPT;
      out->mode_count[k][mode] += 1;
      out->payload_bytes[k] += ltc::rd32(ent + 8);
      out->stream_bytes[k] += len / e;
    }
  }
  return LTC_OK;
}

}  // extern "C"
