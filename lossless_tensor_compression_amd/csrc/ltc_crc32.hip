// ltc_crc32.hip -- per-chunk CRC-32 (zlib's) on gfx950.
//
// cuZipNN 0.1.0 ("API", hash_tensor_with_crc32) defines the checksum as one
// zlib CRC-32 per checksum_chunk_bytes bytes of the buffer, the final piece
// possibly shorter.  One wave per chunk: the chunk is split into 64 lane
// segments, each lane runs a table-driven CRC over its segment with the
// register starting at zero (slicing-by-4 from bank-interleaved tables in
// LDS, ltc_crc.h; Kounavis & Berry, "A Systematic Approach to Building High
// Performance Software-based CRC Generators", 2005), and the 64 partial remainders are
// combined in a 6-level tree whose level l multiplies the left partial by
// x^(8 * seg * 2^l) mod P (the linearity rules are in ltc_crc.h).  A short
// chunk is aligned to the END of its 64-segment frame (leading zero bytes do
// not change a register that starts at zero), so every chunk uses the same
// constants.  zlib's preset is the register value at the chunk's first
// byte, so the lane whose segment holds that byte starts its register at
// 0xFFFFFFFF; the combined register is complemented.
//
// compress_with_crc32 finishes with k_crc_frames: one lane per chunk chains
// the 1 KiB frame remainders that k_scan and k_pack accumulated while they
// wrote the blob (x^(8*1024) multiplications from byte tables in LDS).
#include "ltc_crc.h"
#include "ltc_internal.h"
#include "ltc_launch.h"

namespace ltc {

// The tables take 153 KiB of LDS, so one workgroup of 16 waves holds a CU;
// the grid is at most one workgroup per CU and its waves walk the chunks.
constexpr int kCrcThreads = 1024;
constexpr int kCrcGridMax = 256;
static_assert(kMaxJobs <= 64, "one lane per buffer in k_crc32's prologue");

// DEVLEN: buffer lengths are read on the device (compress_with_crc32).  The
// workgroup then reads each buffer's length once and numbers only the chunks
// that exist (the job table counts chunks of the capacity, about a third
// more for a blob of two thirds of its input).
template <bool DEVLEN>
__global__ __launch_bounds__(kCrcThreads) void k_crc32(CrcArgs a) {
  __shared__ CrcBankLds s;
  __shared__ uint64_t lens[kMaxJobs];         // DEVLEN: the buffers' lengths
  __shared__ uint64_t first[kMaxJobs + 1];    // DEVLEN: their first chunk's index
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64, bl = lane & 31u;
  if (DEVLEN && wave == 0) {  // lane j: buffer j's length and chunk count; their prefix sums
    const uint64_t L = lane < a.count ? *a.jobs[lane].len : 0;
    const uint64_t c = (L + a.chunk_bytes - 1) / a.chunk_bytes;
    uint64_t inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t up = __shfl_up(inc, o, 64);
      if (lane >= (uint32_t)o) inc += up;
    }
    if (lane < a.count) {
      lens[lane] = L;
      first[lane] = inc - c;
    }
    if (lane + 1 == a.count) first[a.count] = inc;
  }
  crc_build_bank(s, a.lvl, tid, kCrcThreads);  // ends with a barrier

  constexpr uint32_t kWaves = kCrcThreads / 64;
  const uint64_t frame = 64 * a.seg;
  const uint64_t total = DEVLEN ? first[a.count] : a.total_chunks;
  int jb = 0;  // a wave's chunk indices only grow, so its buffer index only moves forward
  for (uint64_t gi = (uint64_t)blockIdx.x * kWaves + wave; gi < total; gi += (uint64_t)gridDim.x * kWaves) {
    uint64_t i, len;
    if constexpr (DEVLEN) {
      while (jb + 1 < (int)a.count && gi >= first[jb + 1]) ++jb;
      i = gi - first[jb];
      len = gi + 1 == first[jb + 1] ? lens[jb] - i * a.chunk_bytes : a.chunk_bytes;
    } else {
      while (jb + 1 < (int)a.count && gi >= a.jobs[jb + 1].chunk0) ++jb;
      i = gi - a.jobs[jb].chunk0;
      len = i + 1 == a.jobs[jb].nchunks ? a.jobs[jb].tail_len : a.chunk_bytes;
    }
    const CrcJob& job = a.jobs[jb];
    const uint64_t pad = frame - len;  // leading virtual zero bytes
    const uint64_t vs = lane * a.seg, ve = vs + a.seg;
    const uint8_t* base = job.src + i * a.chunk_bytes;
    const uint8_t* p = base;
    const uint8_t* end = base;
    if (ve > pad) {
      p = base + (vs > pad ? vs - pad : 0);
      end = base + (ve - pad);
    }
    uint32_t crc = vs <= pad && pad < ve ? 0xFFFFFFFFu : 0u;  // zlib's preset at the first byte
    while (p < end && (reinterpret_cast<uintptr_t>(p) & 15)) crc = crc_step1_bank(s, crc, *p++, bl);
    // all sixteen 16-byte loads of a 256-byte segment are in flight together
    for (; p + 256 <= end; p += 256) {
      uint4 q[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) q[u] = reinterpret_cast<const uint4*>(p)[u];
#pragma unroll
      for (int u = 0; u < 16; ++u) crc = crc_step16_bank(s, crc, q[u], bl);
    }
    for (; p + 16 <= end; p += 16) crc = crc_step16_bank(s, crc, *reinterpret_cast<const uint4*>(p), bl);
    for (; p < end; ++p) crc = crc_step1_bank(s, crc, *p, bl);
    crc = crc_tree64_bank(s, crc, lane);
    if (lane == 0) job.out[i] = crc ^ 0xFFFFFFFFu;
  }
}

// One lane per chunk of the blobs' bound.  The register starts at zlib's
// preset at the chunk's first byte and takes in the chunk's frames one by
// one (multiply by x^(8*1024), add the frame's remainder).  The last frame
// of a blob can end past the blob, with zero bytes that no kernel wrote; the
// result is then moved back by those bytes (a multiple of 16).
__global__ __launch_bounds__(256) void k_crc_frames(CrcArgs a) {
  __shared__ uint32_t t1k[4][256];
  __shared__ uint32_t basis[32];
  const uint32_t tid = threadIdx.x;
  if (tid < 32) basis[tid] = gf2_mulmod(1u << tid, a.x1k);
  __syncthreads();
  for (uint32_t idx = tid; idx < 1024; idx += 256) {
    const uint32_t p = idx / 256, b = idx & 255;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b & (1u << i)) v ^= basis[8 * p + i];
    t1k[p][b] = v;
  }
  __syncthreads();
  const uint64_t gi = (uint64_t)blockIdx.x * 256 + tid;
  if (gi >= a.total_chunks) return;
  int jb = 0;
  while (jb + 1 < (int)a.count && gi >= a.jobs[jb + 1].chunk0) ++jb;
  const CrcJob& job = a.jobs[jb];
  const uint64_t i = gi - job.chunk0;
  const uint64_t total = *job.len;
  const uint64_t lo = i * a.chunk_bytes;
  if (lo >= total) return;
  const uint64_t len = min(a.chunk_bytes, total - lo);
  const uint32_t per = (uint32_t)((len + 1023) / 1024);
  const uint32_t* fr = job.frames + lo / 1024;
  auto step = [&](uint32_t c, uint32_t v) {
    return t1k[0][c & 0xFFu] ^ t1k[1][(c >> 8) & 0xFFu] ^ t1k[2][(c >> 16) & 0xFFu] ^
           t1k[3][c >> 24] ^ v;
  };
  uint32_t c = 0xFFFFFFFFu, q = 0;
  for (; q + 8 <= per; q += 8) {  // eight loads in flight
    uint32_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = fr[q + k];
#pragma unroll
    for (int k = 0; k < 8; ++k) c = step(c, v[k]);
  }
  for (; q < per; ++q) c = step(c, fr[q]);
  const uint32_t z = (uint32_t)(1024ull * per - len);
  if (z) c = gf2_mulmod(c, a.xinv[z / 16]);
  job.out[i] = c ^ 0xFFFFFFFFu;
}

hipError_t launch_crc32_frames(const CrcArgs& a, hipStream_t st) {
  if (a.total_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_crc_frames, dim3((uint32_t)((a.total_chunks + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_zero_u32(uint32_t* p, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = 0;
}

hipError_t launch_zero_u32(uint32_t* p, uint64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const uint64_t want = (n + 255) / 256;
  const uint32_t grid = (uint32_t)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(k_zero_u32, dim3(grid), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_crc32(const CrcArgs& a, hipStream_t st) {
  if (a.total_chunks == 0) return hipSuccess;
  const uint64_t want = (a.total_chunks + kCrcThreads / 64 - 1) / (kCrcThreads / 64);
  const uint32_t grid = (uint32_t)(want < kCrcGridMax ? want : kCrcGridMax);
  if (a.jobs[0].len)
    hipLaunchKernelGGL(k_crc32<true>, dim3(grid), dim3(kCrcThreads), 0, st, a);
  else
    hipLaunchKernelGGL(k_crc32<false>, dim3(grid), dim3(kCrcThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ltc
