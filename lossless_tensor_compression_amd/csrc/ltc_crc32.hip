// ltc_crc32.hip -- per-chunk CRC-32 (zlib's) on gfx950.
//
// cuZipNN 0.1.0 ("API", hash_tensor_with_crc32) defines the checksum as the
// zlib CRC-32 of every checksum_chunk_bytes-byte chunk, the last one
// possibly shorter.  One wave per chunk: the chunk is split into 64 lane
// segments, each lane runs a table-driven CRC over its segment with the
// register starting at zero (slicing-by-8 with eight 256-entry tables in LDS;
// Kounavis & Berry, "A Systematic Approach to Building High Performance
// Software-based CRC Generators", 2005), and the 64 partial remainders are
// combined in a 6-level tree.  CRC is linear over GF(2):
//   crc_raw(A || B) = crc_raw(A) * x^(8|B|) mod P  xor  crc_raw(B),
// so each tree level multiplies the left partial by a constant power of x;
// the multiplication by a constant is itself linear and done with four
// 256-entry byte tables per level.  A short chunk is aligned to the END of
// its 64-segment frame (leading zero bytes do not change a register that
// starts at zero), so every chunk uses the same constants.  zlib's initial
// value 0xFFFFFFFF contributes 0xFFFFFFFF * x^(8L) mod P, precomputed for
// the full and the last chunk length, and the result is complemented.
#include "ltc_internal.h"
#include "ltc_launch.h"

namespace ltc {

constexpr uint32_t kPoly = 0xEDB88320u;  // reflected CRC-32 polynomial
constexpr int kCrcThreads = 256;

// a * b mod P with bit 31 - d of a word holding the coefficient of x^d
__device__ __forceinline__ uint32_t gf2_mulmod(uint32_t a, uint32_t b) {
  uint32_t r = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) r ^= b;
    b = (b >> 1) ^ (kPoly & (0u - (b & 1u)));
  }
  return r;
}

__global__ __launch_bounds__(kCrcThreads) void k_crc32(CrcArgs a) {
  __shared__ uint32_t t8[8][256];
  __shared__ uint32_t tl[6][4][256];
  __shared__ uint32_t basis[6][32];
  const uint32_t tid = threadIdx.x;
  {
    // t8[m][b] = CRC register of byte b followed by m zero bytes
    uint32_t c = tid;
    for (int m = 0; m < 8; ++m) {
      for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (kPoly & (0u - (c & 1u)));
      t8[m][tid] = c;
    }
  }
  // multiplication by the level constant is linear: tabulate it per byte
  // position from the images of the 32 single-bit words
  if (tid < 6 * 32) basis[tid / 32][tid % 32] = gf2_mulmod(1u << (tid % 32), a.lvl[tid / 32]);
  __syncthreads();
  for (uint32_t idx = tid; idx < 6 * 4 * 256; idx += kCrcThreads) {
    const uint32_t l = idx / 1024, p = (idx / 256) & 3, b = idx & 255;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b & (1u << i)) v ^= basis[l][8 * p + i];
    tl[l][p][b] = v;
  }
  __syncthreads();

  const uint32_t lane = lane_id(), wave = tid / 64;
  const uint64_t frame = 64 * a.seg;
  for (uint64_t gi = (uint64_t)blockIdx.x * 4 + wave; gi < a.total_chunks;
       gi += (uint64_t)gridDim.x * 4) {
    int jb = 0;
    while (jb + 1 < (int)a.count && gi >= a.jobs[jb + 1].chunk0) ++jb;
    const CrcJob& job = a.jobs[jb];
    const uint64_t i = gi - job.chunk0;
    const bool last = i + 1 == job.nchunks;
    const uint64_t len = last ? job.tail_len : a.chunk_bytes;
    const uint64_t pad = frame - len;  // leading virtual zero bytes
    const uint64_t vs = lane * a.seg, ve = vs + a.seg;
    const uint8_t* base = job.src + i * a.chunk_bytes;
    const uint8_t* p = base;
    const uint8_t* end = base;
    if (ve > pad) {
      p = base + (vs > pad ? vs - pad : 0);
      end = base + (ve - pad);
    }
    uint32_t crc = 0;
    while (p < end && (reinterpret_cast<uintptr_t>(p) & 15)) {
      crc = t8[0][(crc ^ *p) & 0xFFu] ^ (crc >> 8);
      ++p;
    }
    auto step16 = [&](uint32_t c, const uint4 q) {
      c ^= q.x;
      c = t8[7][c & 0xFFu] ^ t8[6][(c >> 8) & 0xFFu] ^ t8[5][(c >> 16) & 0xFFu] ^
          t8[4][c >> 24] ^ t8[3][q.y & 0xFFu] ^ t8[2][(q.y >> 8) & 0xFFu] ^
          t8[1][(q.y >> 16) & 0xFFu] ^ t8[0][q.y >> 24];
      c ^= q.z;
      c = t8[7][c & 0xFFu] ^ t8[6][(c >> 8) & 0xFFu] ^ t8[5][(c >> 16) & 0xFFu] ^
          t8[4][c >> 24] ^ t8[3][q.w & 0xFFu] ^ t8[2][(q.w >> 8) & 0xFFu] ^
          t8[1][(q.w >> 16) & 0xFFu] ^ t8[0][q.w >> 24];
      return c;
    };
    // all sixteen 16-byte loads of a 256-byte segment are in flight together
    for (; p + 256 <= end; p += 256) {
      uint4 q[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) q[u] = reinterpret_cast<const uint4*>(p)[u];
#pragma unroll
      for (int u = 0; u < 16; ++u) crc = step16(crc, q[u]);
    }
    for (; p + 16 <= end; p += 16) crc = step16(crc, *reinterpret_cast<const uint4*>(p));
    for (; p < end; ++p) crc = t8[0][(crc ^ *p) & 0xFFu] ^ (crc >> 8);
#pragma unroll
    for (int l = 0; l < 6; ++l) {
      const uint32_t right = __shfl_down(crc, 1u << l, 64);
      if ((lane & ((2u << l) - 1u)) == 0)
        crc = tl[l][0][crc & 0xFFu] ^ tl[l][1][(crc >> 8) & 0xFFu] ^ tl[l][2][(crc >> 16) & 0xFFu] ^
              tl[l][3][crc >> 24] ^ right;
    }
    if (lane == 0) job.out[i] = crc ^ (last ? job.init_tail : a.init_full) ^ 0xFFFFFFFFu;
  }
}

hipError_t launch_crc32(const CrcArgs& a, hipStream_t st) {
  if (a.total_chunks == 0) return hipSuccess;
  const uint64_t want = (a.total_chunks + 3) / 4;
  const uint32_t grid = (uint32_t)(want < 1280 ? want : 1280);
  hipLaunchKernelGGL(k_crc32, dim3(grid), dim3(kCrcThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace ltc
