// ltc_launch.h -- host-side launchers of the gfx950 kernels.
#pragma once

#include "ltc_internal.h"

namespace ltc {

// Launches k_hist, k_encode, k_scan and k_pack for chunks [t.c_begin,
// t.c_end) on st.  ev (optional): 5 events recorded around the kernels.
// scan_after (optional): the scan waits for it (the previous group's scan);
// scan_done (optional): recorded right after the scan.  staged: the
// histograms and decisions exist already (v2: launch_v2_tables), so k_hist
// and the first two events are left out.
// With t.crc set, k_pack also accumulates the blob's 1 KiB frame remainders
// into each job's frames array (zeroed beforehand with launch_zero_u32).
hipError_t launch_compress(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                           hipEvent_t scan_after = nullptr, hipEvent_t scan_done = nullptr,
                           bool staged = false);

// The same for the top-last layout (t.top_last), in two halves.  Front:
// k_hist (unless staged), k_encode of the lower streams, their scan (after
// scan_after, then scan_done), k_encode of the top streams; events 0-2.
// Back: the top streams' scan (after scan_after, then scan_done) and k_pack;
// events 3-4.  The first group's back half must wait for the last group's
// lower scan: it starts the top streams where the lower ones end.
hipError_t launch_compress_front(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                 hipEvent_t scan_after, hipEvent_t scan_done, bool staged);
hipError_t launch_compress_back(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                hipEvent_t scan_after, hipEvent_t scan_done);

// Format v2 for all chunks of t (c_begin = 0, c_end = total): k_hist (which
// then sums each plane's histograms), k_share (tables, records, payload
// base), k_decide (skip bound per stream).  ev (optional): events 0 and 1.
hipError_t launch_v2_tables(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev);

// p[0, n) = 0 (a kernel, so that the call can be captured in a graph)
hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t st);

// ev (optional): 3 events recorded around the single-table and the
// multi-table decode kernels
hipError_t launch_decompress(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev);

// the same for global chunks [c_begin, c_end) only; init_status: also set
// every job's status to OK first (the first range of a call)
hipError_t launch_decompress_range(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev,
                                   uint64_t c_begin, uint64_t c_end, bool init_status);

struct CrcJob {
  const uint8_t* src;
  uint32_t* out;
  uint64_t chunk0;       // first global chunk index of this buffer
  uint64_t nchunks;      // chunks of the buffer; with len, an upper bound
  uint64_t tail_len;     // length of the buffer's last chunk (without len)
  // optional (all jobs or none): the buffer is its first *len bytes, a length
  // known only on the device (a blob being written); chunks at or past
  // ceil(*len / K) are skipped
  const uint64_t* len;
  // compress_with_crc32: remainders of the buffer's 1 KiB frames, accumulated
  // by k_scan and k_pack while they wrote the blob (k_crc_frames)
  const uint32_t* frames;
};

struct CrcArgs {
  CrcJob jobs[kMaxJobs];
  uint32_t count;
  uint64_t total_chunks;
  uint64_t chunk_bytes;   // K
  uint64_t seg;           // bytes per lane segment (K rounded up to 256, / 64)
  uint32_t lvl[6];        // x^(8*seg*2^l) mod P, reflected
  uint32_t x1k;           // x^(8*1024) mod P
  uint32_t xinv[64];      // x^(-8*16*j) mod P: moves a remainder back by 16*j bytes
};

// whether compress_with_crc32 can combine a K-byte chunk from the 1 KiB
// frame remainders (at most 1024 frames per chunk, chained by one lane)
inline bool crc_frames_usable(uint64_t K) { return K % 1024 == 0 && K <= (1u << 20); }

// k_crc_frames: every chunk of the blobs, one lane per chunk, from the frame
// remainders (jobs need len and frames)
hipError_t launch_crc32_frames(const CrcArgs& a, hipStream_t st);

hipError_t launch_crc32(const CrcArgs& a, hipStream_t st);

}  // namespace ltc

namespace ltc {
inline void record(const hipEvent_t* ev, int i, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev[i], st);
}
}  // namespace ltc
