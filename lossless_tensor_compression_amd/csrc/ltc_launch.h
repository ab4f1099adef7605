// ltc_launch.h -- host-side launchers of the gfx950 kernels.
#pragma once

#include "ltc_internal.h"

namespace ltc {

// Launches k_hist, k_encode, k_scan and k_pack for chunks [t.c_begin,
// t.c_end) on st.  ev (optional): 5 events recorded around the kernels.
// scan_after (optional): the scan waits for it (the previous group's scan);
// scan_done (optional): recorded right after the scan.
// With t.crc set, k_pack also accumulates the blob's 1 KiB frame remainders
// into each job's frames array (zeroed beforehand with launch_zero_u32).
hipError_t launch_compress(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                           hipEvent_t scan_after = nullptr, hipEvent_t scan_done = nullptr);

// p[0, n) = 0 (a kernel, so that the call can be captured in a graph)
hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t st);

// ev (optional): 3 events recorded around the single-table and the
// multi-table decode kernels
hipError_t launch_decompress(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev);

struct CrcJob {
  const uint8_t* src;
  uint32_t* out;
  uint64_t chunk0;       // first global slot of this buffer
  uint64_t nchunks;      // slots of the buffer (see CrcArgs::tail_slot)
  uint64_t tail_len;     // length of the buffer's last chunk (without len)
  uint32_t init_tail;    // 0xFFFFFFFF * x^(8*tail_len) mod P (without len)
  // optional: the buffer is its first *len bytes, a length known only on the
  // device (a blob being written); chunks at or past ceil(*len / K) are skipped
  const uint64_t* len;
  // compress_with_crc32: remainders of the buffer's 1 KiB frames that k_pack
  // accumulated for every byte at or past frames_from, and the number of
  // leading chunks (lead = ceil(frames_from / K)) that hold other bytes too
  const uint32_t* frames;
  uint64_t frames_from;
  uint64_t lead;
};

struct CrcArgs {
  CrcJob jobs[kMaxJobs];
  uint32_t count;
  uint64_t total_chunks;  // slots over all jobs
  uint64_t chunk_bytes;   // K
  uint64_t seg;           // bytes per lane segment (K rounded up to 256, / 64)
  uint32_t lvl[6];        // x^(8*seg*2^l) mod P, reflected
  uint32_t init_full;     // 0xFFFFFFFF * x^(8K) mod P
  uint32_t x1k;           // x^(8*1024) mod P
  // k_crc32 slots: 0 -- slot i is chunk i; 1 -- a job's slots are its `lead`
  // leading chunks and then its last chunk (the chunks k_crc_frames leaves)
  uint32_t tail_slot;
};

// whether compress_with_crc32 can combine a K-byte chunk from k_pack's 1 KiB
// frame remainders (at most 1024 frames per chunk, combined by one lane)
inline bool crc_frames_usable(uint64_t K) { return K % 1024 == 0 && K <= (1u << 20); }

// k_crc_frames: every full chunk at or past a job's lead, except its last,
// combined from the frame remainders (one lane per chunk); a.total_chunks
// then counts chunks of the bound (job.nchunks, job.chunk0 in chunks)
hipError_t launch_crc32_frames(const CrcArgs& a, hipStream_t st);

hipError_t launch_crc32(const CrcArgs& a, hipStream_t st);

}  // namespace ltc

namespace ltc {
inline void record(const hipEvent_t* ev, int i, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev[i], st);
}
}  // namespace ltc
