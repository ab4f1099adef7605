// ltc_internal.h -- device-side types and helpers of the gfx950 codec.
// Not installed; the public contract is include/ltc.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "ltc.h"
#include "ltc_format.h"

namespace ltc {

constexpr uint32_t kModeCand = 0xFF;    // internal: histogram done, encode pending (no blob mode)
constexpr uint32_t kRawStaged = 1;      // internal: a RAW stream's bytes are written (top-last: in
                                        // the blob at their offset; else in the stream's workspace slot)
constexpr uint32_t kPlaced = 2;         // internal: k_encode wrote this RANS payload into the blob
constexpr int kMaxJobs = LTC_BATCH_MAX;

__host__ __device__ constexpr uint64_t align16(uint64_t v) { return (v + 15) & ~uint64_t(15); }

template <int DT> struct Dt;
template <> struct Dt<LTC_U8> { static constexpr int E = 1, WM = -1; };
template <> struct Dt<LTC_BF16> { static constexpr int E = 2, WM = 7; };
template <> struct Dt<LTC_FP16> { static constexpr int E = 2, WM = 10; };
template <> struct Dt<LTC_FP32> { static constexpr int E = 4, WM = 23; };

// Exponent extraction ("NOTE-241: ZipNN", Method item 1): the exponent field
// moves to the top of the element, the sign directly below it, the mantissa
// stays in place.  U8 is the identity.
template <int DT> __device__ __forceinline__ uint32_t reorder(uint32_t x) {
  constexpr int E = Dt<DT>::E, WM = Dt<DT>::WM;
  if constexpr (WM < 0) {
    return x;
  } else {
    constexpr int W = 8 * E, WE = W - 1 - WM;
    const uint32_t e = (x >> WM) & ((1u << WE) - 1u);
    const uint32_t s = (x >> (W - 1)) & 1u;
    return (e << (WM + 1)) | (s << WM) | (x & ((1u << WM) - 1u));
  }
}

// ---------------------------------------------------------------- jobs
// A launch covers up to kMaxJobs tensors of one dtype and chunk size; the
// table travels as a kernel argument.

struct CJob {
  const uint8_t* src;
  const uint8_t* base;        // deltas: XOR base (src's layout), else null
  uint8_t* blob;
  uint64_t* blob_nbytes_out;  // device u64
  uint64_t nbytes;
  uint64_t chunk0;            // first global chunk index of this job
  uint32_t nchunks;
  uint32_t n_tail;            // elements in the last chunk
  uint32_t pmax_full;         // P_max for a full chunk's stream
  uint32_t pmax_tail;         // P_max for the last chunk's stream
  uint32_t* frames;           // with CTable::crc: remainders of the blob's 1 KiB frames
};

struct CTable {
  CJob jobs[kMaxJobs];
  uint32_t count;
  uint32_t chunk_bytes;
  uint32_t n_full;     // elements per full chunk
  uint32_t wcap;       // word capacity per stream in the workspace (multiple of 1024)
  uint64_t total_chunks;
  uint32_t vec16;      // every src 16-byte aligned and chunk_bytes % 16 == 0
  uint32_t dtype;
  uint32_t v2;         // format v2: one table per (tensor, stream index)
  uint32_t delta;      // XOR deltas: every job has a base; ZRUN candidates
  uint32_t top_last;   // layout flag LTC_FLAG_TOP_LAST: stream E-1 of every chunk after the others
  uint32_t place;      // top-last, one group, no deltas: k_encode writes the top streams' RANS
                       // payloads into the blob (offsets from a look-back over CWork::tstat)
  uint64_t place_wait; // with place: device-clock ticks a wave waits for the sizes before it
  // the launch covers global chunks [c_begin, c_end) (a group of a pipelined
  // call, or all of them)
  uint64_t c_begin, c_end;
  // compress_with_crc32: k_scan (header) and k_pack (directory, payloads)
  // accumulate the remainder of every 1 KiB frame of the blob into
  // CJob::frames; k_pack combines runs of frames that lie in one checksum
  // chunk of crc_frames frames
  uint32_t crc;
  uint32_t crc_frames;
  uint32_t crc_x1k;      // x^(8*1024) mod P: one frame on
  uint32_t crc_pos[64];  // x^(8*16*(63-k)) mod P: unit k of a frame to the frame's end
};

struct CWork {
  uint32_t* sinfo;      // [S][4]: size, mode | cval<<8 | lo<<16 | hi<<24, W, 0
  uint16_t* freq;       // [S][256]
  uint32_t* hist;       // v2: [S][256] histograms of the streams to code
  uint64_t* plane;      // v2: [count][E][256] summed histograms (zeroed first)
  uint16_t* ptab;       // v2: [count][E][256] the plane tables
  uint64_t* pbase;      // v2: [count] payload_base (end of the table records)
  uint2* zinfo;         // deltas: [S] nonzero 64-byte blocks, nonzero bytes | rule << 31
  uint32_t* states;     // [S][64]
  uint16_t* words;      // [S][wcap]  (a stream's words end at its slot's end)
  uint64_t* offsets;    // [S]
  uint64_t* blob_nbytes;  // [count] running offset of the scans (top-last: of the lower streams)
  uint64_t* top_run;      // [count] top-last: running offset of the top streams' scan
  uint64_t* tstat;        // CTable::place: [chunks] status of each chunk's top stream (k_encode)
};

struct DJob {
  const uint8_t* blob;
  uint8_t* dst;
  const uint8_t* base;    // deltas: XOR base (dst's layout), else null
  int32_t* status;
  uint64_t payload_base;  // from the header (v1: the end of the directory)
  uint32_t v2;            // table records between the directory and payload_base
  uint32_t top_last;      // header flag LTC_FLAG_TOP_LAST: payload order
  uint64_t blob_nbytes;
  uint64_t nbytes;
  uint64_t chunk0;
  uint32_t nchunks;
  uint32_t n_tail;
};

struct DTable {
  DJob jobs[kMaxJobs];
  uint32_t count;
  uint32_t chunk_bytes;
  uint32_t n_full;
  uint32_t vec16;       // every dst 16-byte aligned and chunk_bytes % 16 == 0
  uint64_t total_chunks;
  uint64_t c_begin;     // a launch decodes global chunks [c_begin, c_end)
  uint64_t c_end;
  uint32_t delta;       // every job is a delta blob with its base
  uint8_t* zbuf;        // deltas: zstride bytes per global stream, ZRUN streams expanded
  uint32_t zstride;     // align16(n_full): a stream's 8-byte reads stay in its slot
};

template <class T>
__device__ __forceinline__ int find_job(const T& t, uint64_t g) {
  int j = 0;
  while (j + 1 < (int)t.count && g >= t.jobs[j + 1].chunk0) ++j;
  return j;
}

// ------------------------------------------------------- wave64 helpers

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Streaming (nontemporal) vector stores, for output no kernel of the call
// reads back.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_nt16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void store_nt8(void* p, uint32_t a, uint32_t b) {
  const u32x2_t v = {a, b};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}

// lane mask of a predicate (the builtin avoids a round trip through a VGPR)
__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// base + lanes_below(mask): mbcnt adds its last operand, which saves the add
__device__ __forceinline__ uint32_t lanes_below_plus(uint64_t mask, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, base));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// exclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_exclusive_scan_u32(uint32_t v) {
  const uint32_t lane = lane_id();
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t up = __shfl_up(inc, o, 64);
    if (lane >= (uint32_t)o) inc += up;
  }
  return inc - v;
}

// Orders LDS accesses across the lanes of one wave (a workgroup of a single
// wave needs no s_barrier): LDS executes a wave's accesses in order, so only
// the compiler must not move them across this point.  Unlike __syncthreads()
// it waits for nothing, in particular not for outstanding global stores.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{})
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

}  // namespace ltc
