// ltc_launch.h -- host-side launchers of the gfx950 kernels.
#pragma once

#include "ltc_internal.h"

namespace ltc {

// Launches k_hist, k_encode, k_scan and k_pack for chunks [t.c_begin,
// t.c_end) on st.  ev (optional): 5 events recorded around the kernels.
// scan_after (optional): the scan waits for it (the previous group's scan);
// scan_done (optional): recorded right after the scan.
hipError_t launch_compress(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                           hipEvent_t scan_after = nullptr, hipEvent_t scan_done = nullptr);

// ev (optional): 3 events recorded around the single-table and the
// multi-table decode kernels
hipError_t launch_decompress(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev);

struct CrcJob {
  const uint8_t* src;
  uint32_t* out;
  uint64_t chunk0;       // first global chunk index of this buffer
  uint64_t nchunks;
  uint64_t tail_len;     // length of the buffer's last chunk
  uint32_t init_tail;    // 0xFFFFFFFF * x^(8*tail_len) mod P
};

struct CrcArgs {
  CrcJob jobs[kMaxJobs];
  uint32_t count;
  uint64_t total_chunks;
  uint64_t chunk_bytes;  // K
  uint64_t seg;          // bytes per lane segment (K rounded up to 256, / 64)
  uint32_t lvl[6];       // x^(8*seg*2^l) mod P, reflected
  uint32_t init_full;    // 0xFFFFFFFF * x^(8K) mod P
};

hipError_t launch_crc32(const CrcArgs& a, hipStream_t st);

}  // namespace ltc

namespace ltc {
inline void record(const hipEvent_t* ev, int i, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev[i], st);
}
}  // namespace ltc
