// ltc_host.h -- host-only parsing of blob bytes (ltc_host.cpp): the header
// check behind ltc_blob_info, the directory walk behind ltc_blob_stats, and
// the split of blobs held in host memory into chunk-ordered copy groups.
// Plain C++ with no HIP, so the code that reads untrusted bytes also builds
// with an ordinary compiler and its address and undefined-behaviour
// sanitizers.
#pragma once

#include <stdint.h>

namespace ltc {

// element size of a dtype code, 0 if unknown
uint32_t elem_bytes(int dtype);

// A blob in host memory as the host-blob decode sees it: `nbytes` bytes at
// `data` whose 64-byte header ltc_blob_info accepted with this blob_nbytes,
// covering global chunks [chunk0, chunk0 + nchunks) of the call; top_last:
// the header's LTC_FLAG_TOP_LAST (payload order).
struct HostBlob {
  const uint8_t* data;
  uint64_t nbytes;
  uint64_t chunk0;
  uint32_t nchunks;
  bool top_last;
};

// One host-to-device copy: bytes [lo, hi) of blob `job`.
struct HostRange {
  uint32_t job;
  uint64_t lo, hi;
};

// Number of copy groups for `total_bytes` of blobs over `total_chunks`
// chunks: about one per group_bytes, at least 1, at most max_groups and at
// most one per chunk (0 when there are no chunks).
uint64_t host_copy_groups(uint64_t total_bytes, uint64_t total_chunks, uint64_t group_bytes,
                          uint64_t max_groups);

// The copies of group g of G (global chunks [T*g/G, T*(g+1)/G)): for every
// blob with a chunk in the group, its bytes from the directory offset of the
// group's first stream in that blob (0 for the blob's first chunk: header
// and directory come along) to the offset of the next group's first stream
// (the blob's end for its last chunk), clamped to [0, nbytes].  A top-last
// blob with E > 1 gives two such ranges: one over its lower streams (ending,
// for its last chunk, at the first top stream) and one over its top streams.
// Reads only the directory entries it needs, each inside [64, payload_base)
// of a blob whose header passed ltc_blob_info.  Writes at most 2 * count
// ranges to out and returns how many.
uint32_t host_group_ranges(const HostBlob* blobs, uint32_t count, uint32_t e, uint64_t T,
                           uint64_t G, uint64_t g, HostRange* out);

}  // namespace ltc
