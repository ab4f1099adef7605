// ltc_compress.hip -- gfx950 compression kernels.
//
// One compress call runs four kernels on the caller's stream:
//   k_hist    one workgroup per chunk: 16-byte loads, exponent-extracting
//             reorder, per-stream 256-bin histograms in LDS (lane-interleaved
//             sub-histograms against same-bin contention), then one wave per
//             stream normalises its histogram to a 4096 total and decides
//             CONST / RAW (by an exact lower bound on the rANS size) / encode.
//   k_encode  one wave per stream index of a chunk still to encode (of two
//             chunks from 16,384 chunks on): 64-lane interleaved rANS from
//             the last step to the first, exact division by one
//             double multiply, words staged in an LDS ring and drained 512
//             bytes at a time to the workspace in decoder order; aborts to
//             RAW as soon as the payload can no longer beat the threshold.
//             The wave coding a top byte also copies the chunk's RAW streams
//             into their workspace slots.
//   k_scan    one workgroup per tensor: exclusive scan of the 16-byte-aligned
//             payload sizes into offsets; writes the 64-byte header.
//   k_pack    one workgroup per chunk: directory entries, RANS payloads and
//             staged RAW streams from the workspace, other RAW streams
//             regrouped from the input; every byte of the blob, padding
//             included, is written exactly once.
// Format v2 (one table per tensor and stream index) puts k_planesum, k_share
// and k_decide between k_hist and k_encode: plane sums of the kept
// histograms, the plane tables, then each stream's skip bound.
// Method: "NOTE-241: ZipNN", Method items 1-3 and 5; chunk size and
// passthrough rule: cuZipNN 0.1.0, API; interleaved rANS lanes and a table per
// stream: lmz README, "On a GPU" and "Building on lmz".
#include <type_traits>

#include "ltc_crc.h"
#include "ltc_internal.h"
#include "ltc_launch.h"

namespace ltc {

constexpr int kHistThreads = 512;
constexpr int kHistCopyShift = 4;
constexpr int kHistCopies = 1 << kHistCopyShift;  // sub-histograms, picked by lane & 15
constexpr uint32_t kHistSeg = 1u << 19;  // elements between sub-histogram flushes
constexpr uint32_t kZSeg = 16384;         // elements per zero bitmap (deltas)
constexpr int kPackThreads = 256;
// CRC variant: a grid of 4 workgroups per CU (13 KiB of tables each, up to
// 128 VGPRs), which build their tables once
constexpr int kPackCrcThreads = 256;
constexpr int kScanThreads = 1024;
constexpr uint32_t kRingWords = 512;    // encoder word ring per stream (LDS)
constexpr uint32_t kFlushWords = 256;   // one drain = 64 lanes x 8 bytes
constexpr int kEncBlock = 8;            // steps per prefetched block (a multiple of 4)
constexpr int kEncStreams = 2;          // streams one wave codes, interleaved (large calls)

__device__ __forceinline__ uint32_t pack_info(uint32_t mode, uint32_t cval, uint32_t lo,
                                              uint32_t hi) {
  return mode | (cval << 8) | (lo << 16) | (hi << 24);
}

// ZRUN payload bytes: 16-byte head, the block bitmap padded to 16, a u64 per
// nonzero 64-byte block padded to 16, the nonzero bytes
__device__ __forceinline__ uint32_t zrun_bytes(uint32_t n, uint32_t nblk, uint32_t nnz) {
  const uint32_t nb = (n + 63) / 64;
  return 16u + (uint32_t)align16((nb + 7) / 8) + (uint32_t)align16(8ull * nblk) + nnz;
}

template <int DT> __device__ __forceinline__ uint32_t load_elem(const uint8_t* p) {
  constexpr int E = Dt<DT>::E;
  if constexpr (E == 1) return *p;
  else if constexpr (E == 2) return *reinterpret_cast<const uint16_t*>(p);
  else return *reinterpret_cast<const uint32_t*>(p);
}

// Deltas ("NOTE-241: ZipNN", Method item 6): the coded element is src XOR
// base, taken at every load so the XOR never touches HBM by itself.
template <int DT, bool DELTA>
__device__ __forceinline__ uint32_t load_x(const uint8_t* src, const uint8_t* base, uint64_t off) {
  uint32_t v = load_elem<DT>(src + off);
  if constexpr (DELTA) v ^= load_elem<DT>(base + off);
  return v;
}

template <bool DELTA>
__device__ __forceinline__ uint4 load_x16(const uint8_t* src, const uint8_t* base, uint64_t off) {
  uint4 v = *reinterpret_cast<const uint4*>(src + off);
  if constexpr (DELTA) {
    const uint4 b = *reinterpret_cast<const uint4*>(base + off);
    v.x ^= b.x;
    v.y ^= b.y;
    v.z ^= b.z;
    v.w ^= b.w;
  }
  return v;
}

// ------------------------------------------------------------------ k_hist

// Sub-histograms: 16 copies, copy = lane & 15, laid out so that the copy
// index picks the LDS bank (word address = (k*128 + bin/2)*16 + copy): 16
// lanes hit 16 different banks whatever their bins.  Two bins share a word as
// 16-bit counters; a copy counts at most kHistSeg/16 = 32768 elements between
// flushes into the 32-bit histogram, so no counter overflows.  16 copies
// rather than 32 halve the LDS of a workgroup (16 KiB), so a CU holds its
// 32-wave limit of them (with 256-thread workgroups: 0.37 against 0.40 ms for
// 1.7 GB of BF16).  512-thread workgroups measured 1-3% faster than 256 on
// calls of 512-1024 chunks and no slower on 13,312; 1024 threads were 5%
// slower there.
template <int DT>
__device__ __forceinline__ void hist_elem(uint32_t* hs, uint32_t y, uint32_t copy) {
  constexpr int E = Dt<DT>::E;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const uint32_t bin = (y >> (8 * k)) & 0xFFu;
    atomicAdd(&hs[((k * 128 + (bin >> 1)) << kHistCopyShift) | copy], 1u << ((bin & 1u) << 4));
  }
}

// one little-endian 32-bit word holds 4/E elements
template <int DT>
__device__ __forceinline__ void hist_word(uint32_t* hs, uint32_t v, uint32_t copy) {
  constexpr int E = Dt<DT>::E;
  if constexpr (E == 4) {
    hist_elem<DT>(hs, reorder<DT>(v), copy);
  } else if constexpr (E == 2) {
    hist_elem<DT>(hs, reorder<DT>(v & 0xFFFFu), copy);
    hist_elem<DT>(hs, reorder<DT>(v >> 16), copy);
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) hist_elem<DT>(hs, (v >> (8 * b)) & 0xFFu, copy);
  }
}

template <int DT>
__device__ __forceinline__ void hist_vec(uint32_t* hs, const uint4 q, uint32_t copy) {
  hist_word<DT>(hs, q.x, copy);
  hist_word<DT>(hs, q.y, copy);
  hist_word<DT>(hs, q.z, copy);
  hist_word<DT>(hs, q.w, copy);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64), hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    v = u > v ? u : v;
  }
  return v;
}

// Frequencies summing to 4096 from counts hv (lane l owns symbols 4l..4l+3,
// n = sum of all counts, at least two nonzero): f = max(1, floor(h*4096/n))
// for h > 0; while the sum exceeds 4096 the largest f > 1 loses one (ties:
// smaller symbol); a shortfall goes to the largest count (ties: smaller
// symbol).  One wave.
template <class T>
__device__ __forceinline__ void normalize_wave(const T hv[4], uint64_t n, uint32_t f[4]) {
  const uint32_t lane = lane_id();
  uint32_t fsum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = hv[i] ? (uint32_t)max((uint64_t)1, ((uint64_t)hv[i] << 12) / n) : 0u;
    fsum += f[i];
  }
  uint32_t total = wave_sum_u32(fsum);
  while (total > kTotal) {  // decrement the largest f > 1, ties to the smaller symbol
    uint32_t key = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (f[i] > 1) key = max(key, (f[i] << 8) | (255u - (4 * lane + i)));
    key = wave_max_u32(key);
    const uint32_t v = 255u - (key & 255u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * lane + i == v) f[i] -= 1;
    --total;
  }
  if (total < kTotal) {  // shortfall to the largest count, ties to the smaller symbol
    uint64_t key = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hv[i]) key = max(key, ((uint64_t)hv[i] << 8) | (255u - (4 * lane + i)));
    key = wave_max_u64(key);
    const uint32_t v = 255u - (uint32_t)(key & 255u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * lane + i == v) f[i] += kTotal - total;
  }
}

// Lower bound on the rANS word count: each coding step gains at least
// log2(4096/f) - log2(16/15) bits of state information (x >= 16 f there),
// each renormalisation loses at most log2(16/15) (x >= 2^20 there), and the
// 64 final states can hold at most 1024 bits more than the initial ones.  If
// even that bound puts the payload (wo + 2 words) above P_max the stream is
// RAW whatever the encoder would do, so it is not encoded.  64 bits of slack
// absorb rounding.
__device__ __forceinline__ bool raw_by_bound(const uint32_t hv[4], const uint32_t f[4], uint32_t n,
                                             uint32_t wo, uint32_t pmax) {
  double bits = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (hv[i]) bits += (double)hv[i] * (12.0 - log2((double)f[i]));
  bits = wave_sum_f64(bits);
  const double wlb = (bits - 0.1862 * (double)n - 1024.0 - 64.0) / 16.0;
  const double plb = (double)wo + 2.0 * (wlb > 0.0 ? ceil(wlb) : 0.0);
  return wo > pmax || plb > (double)pmax;
}

// Normalise one stream's histogram (one wave; lane l owns symbols 4l..4l+3),
// pick CONST / RAW / encode, write the frequency table and the stream info.
// v2 (plane non-null): keep the histogram for k_planesum and k_decide.
__device__ uint32_t normalize_stream(const uint32_t* h, uint32_t n, uint32_t pmax, uint64_t s,
                                     const CWork& w, uint64_t* plane) {
  const uint32_t lane = lane_id();
  uint32_t hv[4], f[4];
  uint32_t nz = 0, lo = 0xFFFFu, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hv[i] = h[4 * lane + i];
    if (hv[i]) {
      ++nz;
      lo = min(lo, 4 * lane + i);
      hi = max(hi, 4 * lane + i);
    }
  }
  nz = wave_sum_u32(nz);
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (plane)  // v2: every stream's histogram, a CONST stream's too, for k_planesum
    *reinterpret_cast<uint4*>(w.hist + 256 * s + 4 * lane) = make_uint4(hv[0], hv[1], hv[2], hv[3]);
  if (nz == 1) {  // a single value: the stream is a header ("NOTE-241", Method item 3)
    if (lane == 0)
      *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = make_uint4(0, pack_info(LTC_MODE_CONST, lo, 0, 0), 0, 0);
    return LTC_MODE_CONST;
  }
  if (plane) {  // v2: decided once the plane's table exists (k_decide)
    if (lane == 0)
      *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = make_uint4(0, pack_info(kModeCand, 0, lo, hi), 0, 0);
    return kModeCand;
  }
  normalize_wave(hv, n, f);
  const uint32_t wo = (uint32_t)align16(kRansFixed + 2u * (hi - lo + 1u));
  const bool raw = raw_by_bound(hv, f, n, wo, pmax);
  const uint64_t packed = (uint64_t)f[0] | ((uint64_t)f[1] << 16) | ((uint64_t)f[2] << 32) |
                          ((uint64_t)f[3] << 48);
  *reinterpret_cast<uint64_t*>(w.freq + 256 * s + 4 * lane) = packed;
  if (lane == 0)
    *reinterpret_cast<uint4*>(w.sinfo + 4 * s) =
        make_uint4(raw ? n : 0u, pack_info(raw ? LTC_MODE_RAW : kModeCand, 0, lo, hi), 0, 0);
  return raw ? LTC_MODE_RAW : kModeCand;
}

// Zero-run statistics of a delta stream (ZipNN's rule, "NOTE-241", Deltas:
// more than 90% zero bytes, or a zero run over 3% of the byte group).  A run
// summary of a range: its length, the zero run at its start and at its end,
// and its longest zero run; summaries of neighbouring ranges join in order.
struct ZRun {
  uint32_t len, pre, suf, mx;
};
__device__ __forceinline__ ZRun zrun_join(ZRun a, ZRun b) {
  ZRun r;
  r.len = a.len + b.len;
  r.pre = a.pre == a.len ? a.len + b.pre : a.pre;
  r.suf = b.suf == b.len ? b.len + a.suf : b.suf;
  r.mx = max(max(a.mx, b.mx), a.suf + b.pre);
  return r;
}

// Run summary of the first L (1..32) flags of x (bit i set: byte i is zero).
__device__ __forceinline__ ZRun zrun_word(uint32_t x, uint32_t L) {
  const uint32_t full = L == 32 ? ~0u : (1u << L) - 1u;
  x &= full;
  if (x == full) return ZRun{L, L, L, L};
  if (x == 0) return ZRun{L, 0, 0, 0};
  uint32_t m = 0;
  for (uint32_t y = x; y; y &= y >> 1) ++m;
  return ZRun{L, (uint32_t)__builtin_ctz(~x), (uint32_t)__builtin_clz(~(x << (32 - L))), m};
}

// Join the lanes' summaries in lane order; lane 0 gets the wave's.
__device__ __forceinline__ ZRun zrun_wave(ZRun z) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    ZRun r;
    r.len = __shfl_down(z.len, o, 64);
    r.pre = __shfl_down(z.pre, o, 64);
    r.suf = __shfl_down(z.suf, o, 64);
    r.mx = __shfl_down(z.mx, o, 64);
    if ((lane & (2 * o - 1)) == 0 && lane + o < 64) z = zrun_join(z, r);
  }
  return z;
}

// Bits of an element x that land in byte k of the reordered element: byte k
// of the reordered element is zero exactly when x & byte_src_mask(k) is.
template <int DT>
__host__ __device__ constexpr uint32_t byte_src_mask(int k) {
  constexpr int E = Dt<DT>::E, WM = Dt<DT>::WM, W = 8 * E;
  uint32_t m = 0;
  for (int b = 0; b < W; ++b) {
    const int to = WM < 0 ? b : (b < WM ? b : (b == W - 1 ? WM : b + 1));
    if (to / 8 == k) m |= 1u << b;
  }
  return m;
}

// Zero flags of stream k for the 16/E elements of a 16-byte vector (bit i:
// element i of the vector).
template <int DT, int K>
__device__ __forceinline__ uint32_t zero_flags(const uint4 q) {
  constexpr int E = Dt<DT>::E, PER = 4 / E;
  const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < PER; ++m)
      bits |= (uint32_t)((wv[i] & (byte_src_mask<DT>(K) << (8 * E * m))) == 0) << (i * PER + m);
  return bits;
}

template <int DT, bool DELTA>
__global__ __launch_bounds__(kHistThreads) void k_hist(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  constexpr uint32_t kWords = E * 128 * kHistCopies;
  // deltas: a zero bitmap per stream for kZSeg elements at a time, whose run
  // summary wave k folds into the stream's before the next slice
  constexpr uint32_t kSub = DELTA ? kZSeg : kHistSeg;
  constexpr uint32_t kZWords = kZSeg / 32;
  __shared__ uint32_t hs[kWords];
  __shared__ uint32_t hf[E * 256];
  __shared__ uint32_t zb[DELTA ? E * kZWords : 1];
  const uint64_t g = t.c_begin + blockIdx.x;
  const int j = find_job(t, g);
  const CJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint8_t* chunk = job.src + c * t.chunk_bytes;
  const uint8_t* bchunk = DELTA ? job.base + c * t.chunk_bytes : nullptr;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const uint32_t copy = tid & (kHistCopies - 1);
  ZRun zacc{0, 0, 0, 0};  // wave k < E, lane 0: stream k so far
  uint32_t nzb = 0;       // nonzero 64-byte blocks of stream k so far

  for (uint32_t i = tid; i < E * 256; i += kHistThreads) hf[i] = 0;
  for (uint32_t seg = 0; seg < n; seg += kHistSeg) {
    const uint32_t sn = n - seg < kHistSeg ? n - seg : kHistSeg;
    for (uint32_t i = tid; i < kWords; i += kHistThreads) hs[i] = 0;
    for (uint32_t sub = 0; sub < sn; sub += kSub) {
      const uint32_t zn = sn - sub < kSub ? sn - sub : kSub;
      const uint32_t len = zn * E;
      const uint8_t* src = chunk + (uint64_t)(seg + sub) * E;
      const uint8_t* bsrc = DELTA ? bchunk + (uint64_t)(seg + sub) * E : nullptr;
      if constexpr (DELTA)
        for (uint32_t i = tid; i < E * kZWords; i += kHistThreads) zb[i] = 0;
      __syncthreads();
      // vector i holds elements [i*16/E, (i+1)*16/E): its zero flags go to
      // bit i*16/E of each stream's bitmap
      auto zvec = [&](const uint4 q, uint32_t i) {
        if constexpr (DELTA) {
          if constexpr (E == 1) {
            reinterpret_cast<uint16_t*>(zb)[i] = (uint16_t)zero_flags<DT, 0>(q);
          } else if constexpr (E == 2) {
            reinterpret_cast<uint8_t*>(zb)[i] = (uint8_t)zero_flags<DT, 0>(q);
            reinterpret_cast<uint8_t*>(zb + kZWords)[i] = (uint8_t)zero_flags<DT, 1>(q);
          } else {
            const uint32_t sh = 4 * (i & 7u);
            atomicOr(&zb[i / 8], zero_flags<DT, 0>(q) << sh);
            atomicOr(&zb[kZWords + i / 8], zero_flags<DT, 1>(q) << sh);
            atomicOr(&zb[2 * kZWords + i / 8], zero_flags<DT, 2>(q) << sh);
            atomicOr(&zb[3 * kZWords + i / 8], zero_flags<DT, 3>(q) << sh);
          }
        }
      };
      uint32_t done = 0;
      if (t.vec16 && len >= 32) {
        const uint32_t nvec = len / 16, lastv = nvec - 1;
        auto v = [&](uint32_t i) { return load_x16<DELTA>(src, bsrc, 16ull * i); };
        // two 16-byte loads in flight ahead of the two being counted; indices
        // are clamped instead of branched so the waits land at the uses
        uint4 q0 = v(min(tid, lastv)), q1 = v(min(tid + kHistThreads, lastv));
        for (uint32_t i = tid; i < nvec; i += 2 * kHistThreads) {
          const uint4 n0 = v(min(i + 2 * kHistThreads, lastv));
          const uint4 n1 = v(min(i + 3 * kHistThreads, lastv));
          hist_vec<DT>(hs, q0, copy);
          zvec(q0, i);
          if (i + kHistThreads < nvec) {
            hist_vec<DT>(hs, q1, copy);
            zvec(q1, i + kHistThreads);
          }
          q0 = n0;
          q1 = n1;
        }
        done = nvec * 16;
      }
      for (uint32_t e = done / E + tid; e < zn; e += kHistThreads) {
        const uint32_t x = load_x<DT, DELTA>(src, bsrc, (uint64_t)e * E);
        hist_elem<DT>(hs, reorder<DT>(x), copy);
        if constexpr (DELTA) {
#pragma unroll
          for (int k = 0; k < E; ++k)
            if ((x & byte_src_mask<DT>(k)) == 0) atomicOr(&zb[k * kZWords + e / 32], 1u << (e & 31u));
        }
      }
      if constexpr (DELTA) {
        __syncthreads();
        if (wave < (uint32_t)E) {  // lane l: words 8l..8l+7 of stream `wave`, four 64-byte blocks
          const uint32_t* zw = zb + wave * kZWords;
          const uint32_t nw = (zn + 31) / 32;
          ZRun z{0, 0, 0, 0};
          uint32_t blocks = 0;
#pragma unroll
          for (uint32_t q = 0; q < kZWords / 64; q += 2) {
            const uint32_t w0 = 8 * lane + q, w1 = w0 + 1;
            if (w0 < nw) {
              const uint32_t l0 = min(32u, zn - 32 * w0);
              const uint32_t m0 = l0 == 32 ? ~0u : (1u << l0) - 1u;
              const uint32_t x0 = zw[w0];
              z = zrun_join(z, zrun_word(x0, l0));
              uint32_t nonzero = ~x0 & m0;
              if (w1 < nw) {
                const uint32_t l1 = min(32u, zn - 32 * w1);
                const uint32_t m1 = l1 == 32 ? ~0u : (1u << l1) - 1u;
                const uint32_t x1 = zw[w1];
                z = zrun_join(z, zrun_word(x1, l1));
                nonzero |= ~x1 & m1;
              }
              blocks += nonzero != 0;
            }
          }
          z = zrun_wave(z);
          blocks = wave_sum_u32(blocks);
          if (lane == 0) {
            zacc = zrun_join(zacc, z);
            nzb += blocks;
          }
        }
        __syncthreads();  // the bitmap is cleared for the next slice
      }
    }
    __syncthreads();
    // fold the copies; the copy index rotates with the thread so the reads
    // of neighbouring lanes hit different banks
    for (uint32_t i = tid; i < E * 256; i += kHistThreads) {
      const uint32_t k = i >> 8, b = i & 255u;
      const uint32_t* row = hs + ((k * 128 + (b >> 1)) << kHistCopyShift);
      const uint32_t sh = (b & 1u) << 4;
      uint32_t sum = 0;
#pragma unroll 8
      for (uint32_t r = 0; r < kHistCopies; ++r) sum += (row[(r + tid) & (kHistCopies - 1)] >> sh) & 0xFFFFu;
      hf[i] += sum;
    }
    __syncthreads();
  }
  __shared__ uint32_t modes[E];
  if (wave < (uint32_t)E) {
    const uint64_t s = g * E + wave;
    const uint32_t pmax = last ? job.pmax_tail : job.pmax_full;
    uint32_t mode = normalize_stream(hf + 256 * wave, n, pmax, s, w,
                                     t.v2 ? w.plane + ((uint64_t)j * E + wave) * 256 : nullptr);
    if constexpr (DELTA) {
      if (lane == 0) {
        // ZipNN's rule makes ZRUN a candidate; k_encode weighs it against
        // RANS, and a stream the size bound made RAW takes it if it fits
        const uint32_t zeros = hf[256 * wave];
        const bool rule = 10ull * zeros > 9ull * n || 100ull * zacc.mx > 3ull * n;
        const uint32_t nnz = n - zeros;
        w.zinfo[s] = make_uint2(nzb, nnz | (rule ? 0x80000000u : 0u));
        if (mode == LTC_MODE_RAW && rule) {
          const uint32_t pz = zrun_bytes(n, nzb, nnz);
          if (pz <= pmax) {
            *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = make_uint4(pz, pack_info(LTC_MODE_ZRUN, 0, 0, 0), nzb, nnz);
            mode = LTC_MODE_ZRUN;
          }
        }
      }
    }
    if (lane == 0) modes[wave] = mode;
  }
  // A coded top byte stages the chunk's RAW streams (see k_encode): its
  // record's third word carries their mask.  The wave that wrote the record
  // adds it, so the two stores keep their order.  v2 decides its streams in
  // k_decide, which sets the mask there.
  if constexpr (E > 1) {
    __syncthreads();
    if (!t.v2 && wave == (uint32_t)(E - 1) && lane == 0 && modes[E - 1] == kModeCand) {
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < E - 1; ++k)
        if (modes[k] == LTC_MODE_RAW) m |= 1u << k;
      if (m) w.sinfo[4 * (g * E + E - 1) + 2] = m;
    }
  }
}

// ---------------------------------------------------------------- v2 tables

__device__ __forceinline__ uint32_t record_bytes(uint32_t lo, uint32_t hi) {
  return lo > hi ? 16u : (uint32_t)align16(16u + 2u * (hi - lo + 1u));
}

// CRC-32 remainder (register from zero) of one 16-byte unit, bit by bit
__device__ __forceinline__ uint32_t unit_remainder_bitwise(uint4 v) {
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
  uint32_t r = 0;
  for (int q = 0; q < 4; ++q)
    for (int b = 0; b < 4; ++b) {
      r ^= (wv[q] >> (8 * b)) & 0xFFu;
      for (int k = 0; k < 8; ++k) r = (r >> 1) ^ (kPoly & (0u - (r & 1u)));
    }
  return r;
}

// v2 plane histograms: thread b sums bin b of stream index k over a block of
// kPlaneBlock chunks (k_hist keeps every stream's histogram in v2) and adds
// each tensor's share to that tensor's plane with one atomic.  The loads of
// a block are independent, so they are in flight together.  Grid:
// E x ceil(chunks / kPlaneBlock).
constexpr uint32_t kPlaneBlock = 16;
template <int DT>
__global__ __launch_bounds__(256) void k_planesum(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  const uint32_t nblk = (uint32_t)((t.total_chunks + kPlaneBlock - 1) / kPlaneBlock);
  const uint32_t k = blockIdx.x / nblk, bin = threadIdx.x;
  uint64_t g = (uint64_t)(blockIdx.x % nblk) * kPlaneBlock;
  const uint64_t g1 = min(g + kPlaneBlock, t.total_chunks);
  while (g < g1) {
    const int j = find_job(t, g);
    const uint64_t gend = min(g1, t.jobs[j].chunk0 + t.jobs[j].nchunks);
    uint64_t acc = 0;
#pragma unroll 8
    for (; g < gend; ++g) acc += w.hist[256 * (g * E + k) + bin];
    if (acc) atomicAdd(reinterpret_cast<unsigned long long*>(w.plane + ((uint64_t)j * E + k) * 256 + bin),
                       (unsigned long long)acc);
  }
}

// One workgroup per tensor, wave k for stream index k: the plane's table
// (the normalised sum of its streams' histograms) into the workspace and as
// a table record into the blob after the directory; payload_base = the end
// of the records.  A plane with at most one value has no table.
template <int DT>
__global__ __launch_bounds__(256) void k_share(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  __shared__ uint32_t rlo[4], rhi[4];
  __shared__ uint16_t sf[4][256];
  const int j = blockIdx.x;
  const CJob& job = t.jobs[j];
  const uint32_t wave = threadIdx.x / 64, lane = lane_id();
  if (wave < (uint32_t)E) {
    const uint64_t* H = w.plane + ((uint64_t)j * E + wave) * 256;
    uint64_t hv[4];
    uint32_t nz = 0, lo = 0xFFFFu, hi = 0;
    uint64_t n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[i] = H[4 * lane + i];
      n += hv[i];
      if (hv[i]) {
        ++nz;
        lo = min(lo, 4 * lane + i);
        hi = max(hi, 4 * lane + i);
      }
    }
    nz = wave_sum_u32(nz);
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += ((uint64_t)__shfl_xor((uint32_t)(n >> 32), o, 64) << 32) | __shfl_xor((uint32_t)n, o, 64);
    uint32_t f[4] = {0, 0, 0, 0};
    if (nz >= 2) normalize_wave(hv, n, f);
    else lo = 1, hi = 0;
    const uint64_t packed = (uint64_t)f[0] | ((uint64_t)f[1] << 16) | ((uint64_t)f[2] << 32) |
                            ((uint64_t)f[3] << 48);
    *reinterpret_cast<uint64_t*>(w.ptab + ((uint64_t)j * E + wave) * 256 + 4 * lane) = packed;
#pragma unroll
    for (int i = 0; i < 4; ++i) sf[wave][4 * lane + i] = (uint16_t)f[i];
    if (lane == 0) {
      rlo[wave] = lo;
      rhi[wave] = hi;
    }
  }
  __syncthreads();
  const uint64_t dir_end = kHeader + kDirEntry * (uint64_t)job.nchunks * E;
  uint64_t off = dir_end, end = dir_end;
  for (int q = 0; q < E; ++q) {
    if ((uint32_t)q < wave) off += record_bytes(rlo[q], rhi[q]);
    end += record_bytes(rlo[q], rhi[q]);
  }
  if (threadIdx.x == 0) w.pbase[j] = end;
  if (wave >= (uint32_t)E) return;
  const uint32_t lo = rlo[wave], hi = rhi[wave];
  const uint32_t units = record_bytes(lo, hi) / 16;
  for (uint32_t u = lane; u < units; u += 64) {
    uint4 v;
    if (u == 0) {
      v = make_uint4(lo | (hi << 16), 0, 0, 0);
    } else {
      uint32_t hw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sym = lo + 8 * (u - 1) + i;
        hw[i] = sym <= hi ? sf[wave][sym] : 0u;
      }
      v = make_uint4(hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16));
    }
    *reinterpret_cast<uint4*>(job.blob + off + 16 * u) = v;
    if (t.crc) {  // this unit's share of its 1 KiB frame (compress_with_crc32)
      const uint64_t ua = (off >> 4) + u;
      const uint32_t r = gf2_mulmod(unit_remainder_bitwise(v), t.crc_pos[ua & 63]);
      if (r) atomicXor(job.frames + (ua >> 6), r);
    }
  }
}

// One wave per stream still to be decided (v2): the skip bound with the
// plane's table; the encoder then codes the rest with that table.
template <int DT>
__global__ __launch_bounds__(256) void k_decide(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  // Each wave decides one stream; the four streams of a workgroup are whole
  // chunks (the launch covers all chunks from chunk 0, four streams per
  // workgroup, E in {1, 2, 4}), so the wave of a chunk's top stream can name
  // the chunk's RAW streams for k_encode to write (as k_hist does in v1).
  __shared__ uint32_t fmode[4];  // each wave's stream: its mode once decided
  const uint32_t wave = threadIdx.x / 64, lane = lane_id();
  const uint64_t s = (t.c_begin * E) + (uint64_t)blockIdx.x * 4 + wave;
  const bool in = s < t.c_end * E;
  uint32_t mode = 0xFFu;
  if (in) {
    const uint32_t info = w.sinfo[4 * s + 1];
    mode = info & 0xFFu;
  }
  if (in && mode == kModeCand) {
    const uint64_t g = s / E;
    const uint32_t k = (uint32_t)(s % E);
    const int j = find_job(t, g);
    const CJob& job = t.jobs[j];
    const bool last = g - job.chunk0 + 1 == job.nchunks;
    const uint32_t n = last ? job.n_tail : t.n_full;
    const uint4 hq = *reinterpret_cast<const uint4*>(w.hist + 256 * s + 4 * lane);
    const uint64_t fq = *reinterpret_cast<const uint64_t*>(w.ptab + ((uint64_t)j * E + k) * 256 + 4 * lane);
    const uint32_t hv[4] = {hq.x, hq.y, hq.z, hq.w};
    const uint32_t f[4] = {(uint32_t)fq & 0xFFFFu, (uint32_t)(fq >> 16) & 0xFFFFu,
                           (uint32_t)(fq >> 32) & 0xFFFFu, (uint32_t)(fq >> 48)};
    const uint32_t pmax = last ? job.pmax_tail : job.pmax_full;
    if (raw_by_bound(hv, f, n, kRansFixed, pmax)) {
      uint4 v = make_uint4(n, pack_info(LTC_MODE_RAW, 0, 0, 0), 0, 0);
      if (t.delta) {  // a delta stream ZipNN's rule fired for: ZRUN if it fits
        const uint2 zi = w.zinfo[s];
        const uint32_t pz = zrun_bytes(n, zi.x, zi.y & 0x7FFFFFFFu);
        if ((zi.y >> 31) && pz <= pmax) v = make_uint4(pz, pack_info(LTC_MODE_ZRUN, 0, 0, 0), zi.x, zi.y & 0x7FFFFFFFu);
      }
      if (lane == 0) *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = v;
      mode = v.y & 0xFFu;
    }
  }
  if constexpr (E > 1) {
    if (lane == 0) fmode[wave] = mode;
    __syncthreads();
    if (in && lane == 0 && s % E == (uint64_t)(E - 1) && mode == kModeCand) {
      uint32_t m = 0;
#pragma unroll
      for (int q = 0; q < E - 1; ++q)
        if (fmode[wave - (E - 1) + q] == LTC_MODE_RAW) m |= 1u << q;
      if (m) w.sinfo[4 * s + 2] = m;
    }
  }
}

// ---------------------------------------------------------------- k_encode

// 24-bit multiply (v_mul_u32_u24, full rate).  The compiler rewrites the
// builtin into a 32-bit multiply whenever it can prove an operand narrow,
// which then issues at quarter rate, so the instruction is named directly.
__device__ __forceinline__ uint32_t mul_u24(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_mul_u32_u24 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Byte k of the reordered element.  For BF16 and FP32 the top byte is the
// biased exponent field itself, one bit-field extract.
template <int DT, bool TOP>
__device__ __forceinline__ uint32_t stream_byte(uint32_t x, uint32_t k) {
  if constexpr (TOP && Dt<DT>::WM >= 0) return (x >> Dt<DT>::WM) & 0xFFu;
  else return (reorder<DT>(x) >> (8 * k)) & 0xFFu;
}

// Byte j of the reordered form of 8 consecutive elements held as loaded (8*E
// bytes, little-endian), packed in element order.  BF16's byte 0 is the low 7
// mantissa bits under the sign: two byte gathers and one bit-field select
// per 4 elements.
template <int DT> __device__ __forceinline__ uint2 stream_bytes8(const uint32_t* pf, int j) {
  constexpr int E = Dt<DT>::E;
  if constexpr (DT == LTC_BF16) {
    // v_perm_b32 selector bytes 0-3 pick bytes of the second operand, 4-7
    // of the first: low and high bytes of the four half-words
    auto four = [](uint32_t w0, uint32_t w1) {
      const uint32_t a = __builtin_amdgcn_perm(w1, w0, 0x06040200u);
      const uint32_t b = __builtin_amdgcn_perm(w1, w0, 0x07050301u);
      return (a & 0x7F7F7F7Fu) | (b & 0x80808080u);
    };
    return make_uint2(four(pf[0], pf[1]), four(pf[2], pf[3]));
  } else {
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t x;
      if constexpr (E == 4) x = pf[i];
      else if constexpr (E == 2) x = (pf[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      else x = (pf[i / 4] >> (8 * (i & 3))) & 0xFFu;
      o[i / 4] |= ((reorder<DT>(x) >> (8 * j)) & 0xFFu) << (8 * (i & 3));
    }
    return make_uint2(o[0], o[1]);
  }
}

// ---- placing the top streams' RANS payloads (top-last layout)
//
// In the top-last layout a tensor's top streams follow its lower streams in
// chunk order, so the payload of chunk g's top stream starts where the lower
// streams end (k_scan part 1) plus the aligned sizes of the top streams of
// the tensor's chunks before g ("NOTE-241: ZipNN", Method item 5: the
// directory says where each payload is; the order is the layout's).  Every
// chunk's top stream has a status word in the workspace: 0 while its size is
// unknown, kStAgg | size once it is coded, kStInc | (bytes of the tensor's top
// streams up to and including it) once that sum is known, and kStLater while
// the 256-entry launch has yet to code it.  k_scan (part 1) sets the status of
// every top stream that needs no coding (its size is final), the tensor's
// first chunk as an inclusive count.  A wave that codes a top stream
// publishes its size, walks back over the statuses of the chunks before it,
// 64 at a time, summing sizes down to the nearest inclusive count, publishes
// its own inclusive count, and writes the payload into the blob itself,
// marking the stream kPlaced so that k_pack skips it.
//
// Waiting.  A wave waits only for chunks with smaller indices, and only after
// publishing its own size.  Workgroups start in index order on each XCD, so
// the lowest-indexed wave not yet started has only running or finished waves
// of lower index on its XCD, which wait for nothing it holds: every chain of
// waits ends at a running wave.  The 128-entry launch runs first and never
// waits for a kStLater chunk (the 256-entry launch codes it later); in the
// 256-entry launch such a chunk belongs to an earlier wave of the launch.
// Every wait is also bounded by the device clock.  A wave that gives up
// leaves its payload to k_pack: the walk decides only who writes the payload
// (offsets, directory and blob size still come from k_scan), so a slow or
// missing status costs time, never a wrong blob.  The status words are the
// only data the waves exchange, so they are read and written with relaxed
// device-scope atomics, coherent across the XCDs' L2 caches without cache
// maintenance (acquire and release forms write back or invalidate the
// XCD's whole L2 at every poll: C3's encoder took 2.47 instead of 0.6 ms).
constexpr uint64_t kStAgg = 1ull << 62, kStInc = 2ull << 62, kStLater = 3ull << 62;
constexpr uint64_t kStVal = (1ull << 62) - 1;

// Bytes of the top streams of chunks [f, g) (f < g: the first chunk of g's
// tensor) from their status words (one wave).  false: a kStLater chunk
// without wait_later, or no answer within `limit` ticks of the device clock.
__device__ bool top_prefix(const uint64_t* st, uint64_t g, uint64_t f, bool wait_later, uint64_t limit,
                           uint64_t& out) {
  const uint32_t lane = lane_id();
  const uint64_t t0 = (uint64_t)wall_clock64();
  uint64_t acc = 0, hi = g;  // chunks [f, hi) are still to add
  while (true) {
    const uint64_t span = hi - f;
    const uint32_t nin = span < 64 ? (uint32_t)span : 64u;  // lane l reads chunk hi - 1 - l
    const bool in = lane < nin;
    const uint64_t v =
        in ? __hip_atomic_load(st + (hi - 1 - lane), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
    const uint64_t fl = v >> 62;
    const uint64_t incm = ballot(in && fl == 2);
    const uint32_t last = incm ? (uint32_t)__builtin_ctzll(incm) : nin - 1;  // the lanes needed: 0..last
    const uint64_t need = last == 63 ? ~0ull : (2ull << last) - 1;
    if (!wait_later && (ballot(in && fl == 3) & need)) return false;
    if ((ballot(in && (fl == 1 || fl == 2)) & need) != need) {
      if ((uint64_t)wall_clock64() - t0 > limit) return false;
      __builtin_amdgcn_s_sleep(4);
      continue;  // read the window again
    }
    acc += wave_sum_u64(lane <= last ? (v & kStVal) : 0ull);
    if (incm || span <= 64) {
      out = acc;
      return true;
    }
    hi -= 64;
  }
}

// bytes [sh, sh + 16) of the 32 bytes a, b (sh even, below 16)
__device__ __forceinline__ uint4 shift_blocks(const uint4 a, const uint4 b, uint32_t sh) {
  const uint32_t q = sh >> 2;
  const uint32_t w0 = q == 0 ? a.x : q == 1 ? a.y : q == 2 ? a.z : a.w;
  const uint32_t w1 = q == 0 ? a.y : q == 1 ? a.z : q == 2 ? a.w : b.x;
  const uint32_t w2 = q == 0 ? a.z : q == 1 ? a.w : q == 2 ? b.x : b.y;
  const uint32_t w3 = q == 0 ? a.w : q == 1 ? b.x : q == 2 ? b.y : b.z;
  if (!(sh & 2u)) return make_uint4(w0, w1, w2, w3);
  const uint32_t w4 = q == 0 ? b.x : q == 1 ? b.y : q == 2 ? b.z : b.w;
  return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, 2), __builtin_amdgcn_alignbyte(w2, w1, 2),
                    __builtin_amdgcn_alignbyte(w3, w2, 2), __builtin_amdgcn_alignbyte(w4, w3, 2));
}

// One wave codes stream k of U neighbouring chunks: in large calls two,
// interleaving their independent state chains (instruction-level parallelism
// for a loop whose every step is a dependent chain), in smaller ones one
// (more waves in flight; see launch_encode).
//
// Division.  A coding step needs q = floor(x / f) for a 32-bit x and
// 1 <= f <= 4095.  With r = 1/f rounded up to a double, x * r >= x / f, and
// the excess x/f * 2^-52 < 2^-20, while a non-integral x/f sits at least 1/f
// >= 2^-12 below the next integer; so truncating the rounded product gives q
// exactly (rounding is monotone and q is representable).  The same quotient
// decides renormalisation: x >= f * 2^20 exactly when floor(x / f) >= 2^20,
// and then floor((x >> 16) / f) = floor(x / f) >> 16.
//
// Per stream, in LDS:
//   tab   one 16-byte entry per symbol: {r (double), 4096 - f, cum}.  A
//         second instantiation holds 128 entries from the stream's lowest
//         symbol and takes the waves whose coded streams all span at most
//         128 symbols (exponent streams of trained weights span about 40):
//         with two streams a wave, its 8,448 bytes of LDS let 16 waves share
//         a CU (then the 99 VGPRs bound it) instead of 12, and the encoder
//         ran about 7% faster.  Both are launched; each leaves the other's
//         waves alone.
//   stg   one block of 512 elements, loaded with wide coalesced loads one
//         block ahead, stored as their symbols' table offsets and read back
//         transposed to lane order;
//   ring  512 emitted words.  The words of a step take decoder order (lanes
//         ascending), so lane l's word lands at top - cnt + (number of
//         emitting lanes below l); complete 256-word blocks drain to the
//         workspace with 8-byte stores, and a stream's words end at the end
//         of its workspace slot.
// Abort and drain checks run every 4 steps: 4 steps emit at most 256 words,
// so a block is never overwritten before it drains, and an abort is seen
// before any word past the stream's limit reaches the workspace.
//
// Staging.  The wave coding a chunk's top byte loads every byte of its
// elements, so it also writes the chunk's RAW streams (those k_hist decided,
// named in its record's third word).  In the top-last layout their blob
// offsets are known by then (the lower streams are scanned before the top
// streams are coded), so the bytes go straight to their place in the blob;
// otherwise they go, in blob order, into the streams' own workspace slots,
// which nothing else uses, and k_pack copies them instead of regrouping the
// input again.  Only whole chunks of full 8-step blocks coded in lock step
// are staged, and a stream is marked staged (fourth word of its record) once
// every block is written and the top stream was not abandoned; k_pack writes
// the others whole.
//
// A launch codes the stream indices kfirst, kfirst - 1, ... (nplanes of
// them): all E at once, or in the top-last layout the lower ones and then,
// after their scan, the top one.
template <int DT, bool DELTA, int TABN, int U>
__global__ __launch_bounds__(64) void k_encode(CTable t, CWork w, uint32_t kfirst, uint32_t nplanes) {
  constexpr int E = Dt<DT>::E;
  __shared__ uint4 tab[U][TABN];
  __shared__ __attribute__((aligned(16))) uint32_t stg[U][256];  // 512 u16 entry offsets
  __shared__ __attribute__((aligned(16))) uint16_t ring[U][kRingWords];
  const uint32_t lane = lane_id();
  // Stream-index-major order, the top byte (usually the only coded stream)
  // first: consecutive workgroups go to different XCDs in turn, so
  // interleaving the stream indices would hand every coded stream of a
  // BF16 tensor to half of the XCDs (of an FP32 tensor, to a quarter) while
  // the rest only receive streams that exit at once.
  // Deltas usually code every stream of a chunk, and each wave reads whole
  // elements of source and base: there the E workgroups of a wave's chunks
  // sit 8 apart (blocks of 8), so they reach the same XCD together and walk
  // the same elements in the same order, and the later reads hit its L2.
  // The launch rounds the grid up to whole blocks; the spare workgroups find
  // no chunk and exit.
  uint32_t k;
  uint64_t g0;
  if constexpr (DELTA) {
    const uint32_t grp = blockIdx.x / (8u * nplanes), r = blockIdx.x % (8u * nplanes);
    k = kfirst - r / 8u;
    g0 = t.c_begin + (uint64_t)(grp * 8u + r % 8u) * U;
  } else {
    const uint32_t per_plane = gridDim.x / nplanes;  // workgroups per stream index
    k = kfirst - blockIdx.x / per_plane;
    g0 = t.c_begin + (uint64_t)(blockIdx.x % per_plane) * U;
  }
  const uint32_t wcap = t.wcap;

  bool on[U];
  uint64_t sid[U];
  uint32_t n[U], full[U], wlimit[U], wo[U], lo[U], hi[U], smask[U];
  const uint8_t* src[U];
  const uint8_t* bsrc[U];
  const uint16_t* ftab[U];
  uint4 fallback[U];  // the stream's directory info if coding it does not pay
  int jb[U];          // the chunk's tensor
  uint8_t* rdst[U][E > 1 ? E - 1 : 1];  // where staged RAW stream j of the chunk goes
#pragma unroll
  for (int u = 0; u < U; ++u) {
    on[u] = false;
    sid[u] = 0;
    n[u] = full[u] = wlimit[u] = wo[u] = lo[u] = hi[u] = smask[u] = 0;
    src[u] = nullptr;
    bsrc[u] = nullptr;
    ftab[u] = nullptr;
    fallback[u] = make_uint4(0, 0, 0, 0);
    jb[u] = 0;
#pragma unroll
    for (int q = 0; q < (E > 1 ? E - 1 : 1); ++q) rdst[u][q] = nullptr;
    const uint64_t g = g0 + u;
    if (g >= t.c_end) continue;
    const uint64_t s = g * E + k;
    const uint32_t info = w.sinfo[4 * s + 1];
    if ((info & 0xFFu) != kModeCand) continue;
    const int j = find_job(t, g);
    const CJob& job = t.jobs[j];
    const uint64_t c = g - job.chunk0;
    const bool last = c + 1 == job.nchunks;
    on[u] = true;
    jb[u] = j;
    sid[u] = s;
    n[u] = last ? job.n_tail : t.n_full;
    full[u] = n[u] / 64;
    lo[u] = (info >> 16) & 0xFFu;
    hi[u] = info >> 24;
    if (E > 1 && k == (uint32_t)(E - 1) && n[u] % (64u * kEncBlock) == 0 && n[u] <= 2u * wcap) {
      smask[u] = w.sinfo[4 * s + 2];
#pragma unroll
      for (int q = 0; q < E - 1; ++q)
        if (smask[u] & (1u << q))
          rdst[u][q] = t.top_last ? job.blob + w.offsets[s - k + q]
                                  : reinterpret_cast<uint8_t*>(w.words + (s - k + q) * wcap);
    }
    // v2: the plane's table and no table in the payload
    wo[u] = t.v2 ? kRansFixed : (uint32_t)align16(kRansFixed + 2u * (hi[u] - lo[u] + 1u));
    ftab[u] = t.v2 ? w.ptab + ((uint64_t)j * E + k) * 256 : w.freq + 256 * s;
    const uint32_t pmax = last ? job.pmax_tail : job.pmax_full;
    uint32_t limit = pmax;
    fallback[u] = make_uint4(n[u], pack_info(LTC_MODE_RAW, 0, 0, 0), 0, 0);
    if constexpr (DELTA) {
      // a ZRUN candidate (the zero-run rule fired): RANS must also be no
      // larger than it; otherwise ZRUN if within P_max, else RAW
      const uint2 zi = w.zinfo[s];
      if (zi.y >> 31) {
        const uint32_t pz = zrun_bytes(n[u], zi.x, zi.y & 0x7FFFFFFFu);
        if (pz <= pmax) {
          limit = pz;
          fallback[u] = make_uint4(pz, pack_info(LTC_MODE_ZRUN, 0, 0, 0), zi.x, zi.y & 0x7FFFFFFFu);
        }
      }
      if (limit < wo[u]) {  // no RANS payload fits
        on[u] = false;
        if (lane == 0) *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = fallback[u];
        continue;
      }
      bsrc[u] = job.base + c * t.chunk_bytes;
    }
    wlimit[u] = (limit - wo[u]) / 2;
    src[u] = job.src + c * t.chunk_bytes;
  }
  {
    bool any = false;
#pragma unroll
    for (int u = 0; u < U; ++u) any = any || on[u];
    if (!any) return;
  }
  // the short-table instantiation takes the waves whose coded streams use at
  // most TABN consecutive symbols (filled from the stream's lowest symbol, v1
  // or v2 tables alike); the full one the others
  {
    bool small = true;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (on[u] && hi[u] - lo[u] >= 128u) small = false;
    if (small != (TABN < 256)) {
      // placement: the 128-entry launch runs first and marks the top streams
      // it leaves to the 256-entry one, so that no wave of it waits for them
      if (TABN < 256 && t.place && k == (uint32_t)(E - 1) && lane == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) __hip_atomic_store(w.tstat + g0 + u, kStLater, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
  }
  bool mine[U];  // the top streams this wave codes (placement)
#pragma unroll
  for (int u = 0; u < U; ++u) mine[u] = on[u];
  uint32_t toff[U];  // the symbol of table entry 0
#pragma unroll
  for (int u = 0; u < U; ++u) toff[u] = TABN < 256 ? lo[u] : 0u;

#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!on[u]) continue;
    const uint64_t fq = *reinterpret_cast<const uint64_t*>(ftab[u] + 4 * lane);
    uint32_t f[4], cum[4], acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (uint32_t)(fq >> (16 * i)) & 0xFFFFu;
      cum[i] = acc;
      acc += f[i];
    }
    const uint32_t base = wave_exclusive_scan_u32(acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double r = 0.0;
      if (f[i]) {
        const double fd = (double)f[i];
        r = 1.0 / fd;                                  // correctly rounded
        if (fma(r, fd, -1.0) < 0.0)                    // below 1/f: one ulp up
          r = __longlong_as_double(__double_as_longlong(r) + 1);
      }
      const uint64_t rb = (uint64_t)__double_as_longlong(r);
      const uint32_t slot = 4 * lane + i - toff[u];  // wraps past TABN for symbols below toff
      if (slot < (uint32_t)TABN)
        tab[u][slot] = make_uint4((uint32_t)rb, (uint32_t)(rb >> 32), kTotal - f[i], base + cum[i]);
    }
  }
  __syncthreads();

  // Words emitted so far: wcap - top.  A stream aborts once top < atop
  // (more than wlimit words) and drains the 256 words at [ftop, ftop + 256)
  // once top <= ftop.
  uint32_t x[U], top[U], ftop[U], atop[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    x[u] = kRansLow;
    top[u] = wcap;
    ftop[u] = wcap - kFlushWords;
    atop[u] = wcap - wlimit[u];
  }

  auto flush = [&](int u) {
    wave_sync();  // the block's words were written by other lanes
    const uint32_t base = ftop[u] + 4 * lane;
    const uint2 v = *reinterpret_cast<const uint2*>(&ring[u][base & (kRingWords - 1)]);
    *reinterpret_cast<uint2*>(w.words + sid[u] * wcap + base) = v;
  };
  // Every 4 steps: 4 steps emit at most 256 words, so at most one block is
  // complete and none is overwritten before it drains.
  auto check = [&](int u) {
    if (top[u] < atop[u]) {
      on[u] = false;
      if (lane == 0) *reinterpret_cast<uint4*>(w.sinfo + 4 * sid[u]) = fallback[u];
    } else if (top[u] <= ftop[u]) {
      flush(u);
      ftop[u] = uniform(ftop[u] - kFlushWords);
    }
  };
  // One coding step of stream u (steps run from the last to the first).
  // Only emitting lanes write the ring, under an exec mask: the ring byte
  // offset comes from mbcnt and one shift-add of the uniform top, with no
  // private slot to select (C2 compress 0.108 -> 0.105 ms, C5 1% faster).
  auto code = [&](auto guarded, int u, const uint4 e) {
    constexpr bool G = decltype(guarded)::value;
    const bool active = !G || lane < (n[u] & 63u);
    const uint32_t xo = x[u];
    const double r = __hiloint2double((int)e.y, (int)e.x);
    const uint32_t q1 = (uint32_t)((double)xo * r);
    const bool need = active && q1 >= (1u << 20);
    const uint64_t mask = ballot(need);
    const uint32_t sh = need ? 16u : 0u;
    const uint32_t xn = mul_u24(q1 >> sh, e.z) + (xo >> sh) + e.w;
    x[u] = active ? xn : xo;
    top[u] = uniform(top[u] - (uint32_t)__popcll(mask));
    if (need) {  // the emitting lanes only (an exec mask); the ring position in bytes
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
      const uint32_t off = ((below << 1) + 2u * top[u]) & (2u * kRingWords - 2u);
      *reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ring[u]) + off) = (uint16_t)xo;
    }
  };

  auto body = [&](auto topexp) {
    constexpr bool TOP = decltype(topexp)::value;
    auto sym_at = [&](int u, uint32_t step) -> uint32_t {  // direct load, index clamped
      const uint32_t e = 64 * step + lane;
      return stream_byte<DT, TOP>(
          load_x<DT, DELTA>(src[u], bsrc[u], (uint64_t)(e < n[u] ? e : n[u] - 1) * E), k);
    };
    // the partial step (the last one) is coded first
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (on[u] && n[u] > 64 * full[u]) {
        code(std::true_type{}, u, tab[u][sym_at(u, full[u]) - toff[u]]);
        check(u);
      }
    }
    // Fast loop: both streams have the same number of full steps (the common
    // case) and code them in lock step, 8 steps (512 elements per stream) per
    // block.  Each lane loads 8*E contiguous bytes of the next block with one
    // wide load, the block goes through the LDS tile, and every lane reads
    // back its own element of each step at a fixed offset.
    uint32_t done = 0;  // full steps coded, counted from the last one down
    bool lock = t.vec16 != 0;
#pragma unroll
    for (int u = 0; u < U; ++u) lock = lock && on[u] && full[u] == full[0];
    const uint32_t nfb = lock ? full[0] / kEncBlock : 0u;
    uint32_t pf[U][2 * E];
    auto fetch = [&](int u, uint32_t bi) {  // block bi: elements 64*(full - 8(bi+1)) + 8 lane ...
      const uint32_t e0 = 64u * (full[u] - kEncBlock * (bi + 1)) + 8u * lane;
      if constexpr (E == 1) {
        uint2 v = *reinterpret_cast<const uint2*>(src[u] + e0);
        if constexpr (DELTA) {
          const uint2 b = *reinterpret_cast<const uint2*>(bsrc[u] + e0);
          v.x ^= b.x;
          v.y ^= b.y;
        }
        pf[u][0] = v.x;
        pf[u][1] = v.y;
      } else {
#pragma unroll
        for (int h = 0; h < E / 2; ++h) {
          const uint4 v = load_x16<DELTA>(src[u], bsrc[u], (uint64_t)e0 * E + 16 * h);
          pf[u][4 * h] = v.x;
          pf[u][4 * h + 1] = v.y;
          pf[u][4 * h + 2] = v.z;
          pf[u][4 * h + 3] = v.w;
        }
      }
    };
    // The tile holds, per element, the byte offset of its symbol's table
    // entry (symbol * 16) as a u16: the steps then read their entry address
    // straight from LDS.
    auto entry_offsets = [&](int u) -> uint4 {
      uint32_t o[4];
      if constexpr (DT == LTC_BF16 && TOP) {
        // the exponent of each half-word sits in bits 7..14: (x >> 3) & 0xFF0
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (pf[u][i] >> 3) & 0x0FF00FF0u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t a, b;
          if constexpr (E == 1) {
            a = ((pf[u][i >> 1] >> (16 * (i & 1))) & 0xFFu) << 4;
            b = ((pf[u][i >> 1] >> (16 * (i & 1) + 8)) & 0xFFu) << 4;
          } else if constexpr (E == 2) {
            a = stream_byte<DT, TOP>(pf[u][i] & 0xFFFFu, k) << 4;
            b = stream_byte<DT, TOP>(pf[u][i] >> 16, k) << 4;
          } else {
            a = stream_byte<DT, TOP>(pf[u][2 * i], k) << 4;
            b = stream_byte<DT, TOP>(pf[u][2 * i + 1], k) << 4;
          }
          o[i] = a | (b << 16);
        }
      }
      // entry offsets from the table's first symbol (every symbol is >= it,
      // so neither half borrows)
      const uint32_t d = (toff[u] << 4) * 0x10001u;
      return make_uint4(o[0] - d, o[1] - d, o[2] - d, o[3] - d);
    };
    // Software pipeline, per block of 8 steps: the entries of a half-block's
    // 4 steps are read while the previous 4 steps compute, and the next block
    // is staged (and the one after it loaded) between the two halves, so the
    // state chains never wait on LDS or HBM.  A tile staged past the last
    // block repeats in-bounds data and is never coded.
    auto stage = [&]() {
      wave_sync();
#pragma unroll
      for (int u = 0; u < U; ++u) reinterpret_cast<uint4*>(stg[u])[lane] = entry_offsets(u);
      wave_sync();
    };
    // step full-1-8bi-q sits at element 64*(7-q) + lane of the tile
    auto read_offsets = [&](uint32_t (&sy)[U][kEncBlock]) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < kEncBlock; ++q)
          sy[u][q] = reinterpret_cast<const uint16_t*>(stg[u])[64 * (kEncBlock - 1 - q) + lane];
    };
    auto entry_at = [&](int u, uint32_t off) {
      return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(tab[u]) + off);
    };
    // RAW stream bytes of the block in pf, taken when it is staged and
    // stored after the next block's loads are issued
    uint2 rw[U][E > 1 ? E - 1 : 1];
    auto raw_take = [&]() {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < E - 1; ++j)
          if (smask[u] & (1u << j)) rw[u][j] = stream_bytes8<DT>(pf[u], j);
    };
    auto raw_put = [&](uint32_t bi) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < E - 1; ++j)
          if (smask[u] & (1u << j)) {  // a uniform block address and a lane offset
            uint8_t* blk = rdst[u][j] + 64u * (full[u] - kEncBlock * (bi + 1));
            *reinterpret_cast<uint2*>(blk + 8u * lane) = rw[u][j];
          }
    };
    if (nfb > 0) {
      uint32_t sy[U][kEncBlock], sn[U][kEncBlock];
      uint4 ta[U][4], tb[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) fetch(u, 0);
      stage();
      raw_take();
      read_offsets(sy);
#pragma unroll
      for (int u = 0; u < U; ++u) fetch(u, nfb > 1 ? 1u : 0u);
      raw_put(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) ta[u][q] = entry_at(u, sy[u][q]);
      for (uint32_t bi = 0; bi < nfb; ++bi) {
        // steps 0..3 of the block; the entries of steps 4..7 load meanwhile
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            code(std::false_type{}, u, ta[u][q]);
            tb[u][q] = entry_at(u, sy[u][4 + q]);
          }
        }
        // stage block bi+1 (loaded one block ago), load block bi+2; the
        // drain check comes after, so its stores are a half-block old by the
        // time the next staging waits on the loads (one counter covers both)
        stage();
        raw_take();
        read_offsets(sn);
        const uint32_t nxt = bi + 2 < nfb ? bi + 2 : nfb - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) fetch(u, nxt);
        if (bi + 1 < nfb) raw_put(bi + 1);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) check(u);
        // steps 4..7; the entries of the next block's steps 0..3 load meanwhile
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            code(std::false_type{}, u, tb[u][q]);
            ta[u][q] = entry_at(u, sn[u][q]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) check(u);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < kEncBlock; ++q) sy[u][q] = sn[u][q];
        done = kEncBlock * (bi + 1);
        bool all = true;
#pragma unroll
        for (int u = 0; u < U; ++u) all = all && on[u];
        if (!all) break;  // the survivor finishes below
      }
    }
    // General path: whatever the fast loop left (streams of different
    // lengths, unaligned inputs, the last full % 8 steps, the partner of a
    // stream that aborted), one step at a time with direct element loads.
    uint32_t rest = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) rest = max(rest, on[u] ? full[u] - done : 0u);
    for (uint32_t i = 0; i < rest; ++i) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (on[u] && done + i < full[u])
          code(std::false_type{}, u, tab[u][sym_at(u, full[u] - 1 - done - i) - toff[u]]);
      if ((i & 3) == 3) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (on[u]) check(u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!on[u]) continue;
      check(u);
      if (!on[u]) continue;
      const uint32_t nw = wcap - top[u];
      if (top[u] < ftop[u] + kFlushWords) flush(u);  // the last, partial block
      // the fast loop staged every block and the stream was kept: lane j
      // marks RAW stream j of the chunk staged
      if (smask[u] && done == full[u] && lane < (uint32_t)(E - 1) && (smask[u] & (1u << lane)))
        w.sinfo[4 * (sid[u] - k + lane) + 3] = kRawStaged;
      w.states[64 * sid[u] + lane] = x[u];
      if (lane == 0)
        *reinterpret_cast<uint4*>(w.sinfo + 4 * sid[u]) =
            make_uint4(wo[u] + 2 * nw, pack_info(LTC_MODE_RANS, 0, lo[u], hi[u]), nw, 0);
    }
  };
  const bool topexp = (DT == LTC_BF16 || DT == LTC_FP32) && k == (uint32_t)(E - 1);
  if (topexp) body(std::true_type{});
  else body(std::false_type{});

  if constexpr (!DELTA) {
    if (!t.place || k != (uint32_t)(E - 1)) return;
    // sizes first (a coded stream's payload, or the RAW fallback of one
    // that did not pay), then each stream's walk
    uint64_t fsz[U], pre[U];
    bool got[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      got[u] = false;
      fsz[u] = pre[u] = 0;
      if (!mine[u]) continue;
      fsz[u] = align16(on[u] ? wo[u] + 2ull * (wcap - top[u]) : (uint64_t)fallback[u].x);
      const bool first = g0 + u == t.jobs[jb[u]].chunk0;
      if (lane == 0)
        __hip_atomic_store(w.tstat + g0 + u, (first ? kStInc : kStAgg) | fsz[u], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    // ticks of the 100 MHz device clock (the host sets 1 ms plus 20 ns per
    // element of a chunk, several times the coding time of a stream; 0 with
    // LTC_FLAG_PLACE_NO_WAIT: give up at the first unknown size)
    const uint64_t limit = t.place_wait;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!mine[u]) continue;
      const uint64_t g = g0 + u, f = t.jobs[jb[u]].chunk0;
      if (g == f) {
        got[u] = true;
      } else if (u > 0 && mine[u - 1] && got[u - 1] && jb[u - 1] == jb[u]) {
        pre[u] = pre[u - 1] + fsz[u - 1];
        got[u] = true;
      } else {
        got[u] = top_prefix(w.tstat, g, f, TABN == 256, limit, pre[u]);
      }
      if (got[u] && g != f && lane == 0)
        __hip_atomic_store(w.tstat + g, kStInc | (pre[u] + fsz[u]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the payloads: prefix, the 64 final states, v1's table, the words from
    // the stream's workspace slot (the drains of this wave; the slot ends on
    // a 16-byte boundary, so they are read as aligned blocks shifted into
    // place, blocks past the end as zeros) and zeros to the next 16 bytes.
    // The words were stored by other lanes of this one-wave workgroup: a
    // workgroup-scope fence orders them before the loads.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!got[u] || !on[u]) continue;
      const uint32_t nw = wcap - top[u];
      uint8_t* dst = t.jobs[jb[u]].blob + w.blob_nbytes[jb[u]] + pre[u];
      if (lane == 0) *reinterpret_cast<uint4*>(dst) = make_uint4(nw, t.v2 ? 0u : lo[u] | (hi[u] << 8), 0u, 0u);
      reinterpret_cast<uint32_t*>(dst + 16)[lane] = x[u];
      const uint32_t tcount = t.v2 ? 0u : hi[u] - lo[u] + 1u;
      const uint16_t* fr = w.freq + 256 * sid[u] + lo[u];
      for (uint32_t i = lane; i < (wo[u] - kRansFixed) / 2; i += 64)
        reinterpret_cast<uint16_t*>(dst + kRansFixed)[i] = i < tcount ? fr[i] : (uint16_t)0;
      const uint8_t* ws = reinterpret_cast<const uint8_t*>(w.words + sid[u] * wcap + (wcap - nw));
      const uint32_t sh = (uint32_t)(reinterpret_cast<uintptr_t>(ws) & 15u);
      const uint4* ab = reinterpret_cast<const uint4*>(ws - sh);
      const uint32_t nsrc = (sh + 2u * nw) / 16u, wunits = (2u * nw + 15u) / 16u;
      uint4* wd = reinterpret_cast<uint4*>(dst + wo[u]);
      for (uint32_t i0 = lane; i0 < wunits; i0 += 256) {
        uint4 va[4], vb[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // clamped loads, then selects (block i < wunits <= nsrc)
          const uint32_t i = i0 + 64 * q;
          const uint4 a = ab[min(i, wunits - 1u)], b = ab[min(i + 1u, nsrc - 1u)];
          va[q] = i < wunits ? a : z;
          vb[q] = sh && i + 1 < nsrc ? b : z;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t i = i0 + 64 * q;
          if (i < wunits) wd[i] = shift_blocks(va[q], vb[q], sh);
        }
      }
      if (lane == 0) w.sinfo[4 * sid[u] + 3] = kPlaced;
    }
  }
}

// ------------------------------------------------------------------ k_scan

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_up((uint32_t)v, o, 64);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

// One workgroup per tensor: exclusive scan of the 16-byte-aligned payload
// sizes of the tensor's streams inside this launch's chunk range, in blob
// order.  part 0: every stream (directory order); top-last layout: part 1
// the lower streams k < E-1 (directory order), part 2 the top streams (chunk
// order), which start where the tensor's last lower stream ends.  A
// pipelined call scans its groups in chunk order; the running offset passes
// from one group to the next through blob_nbytes[j] (parts 0 and 1) or
// top_run[j] (part 2), and the group holding the tensor's last chunk writes
// the blob size and the header (parts 0 and 2).
__global__ __launch_bounds__(kScanThreads) void k_scan(CTable t, CWork w, uint32_t E, uint32_t part) {
  __shared__ uint64_t wave_tot[kScanThreads / 64];
  const int j = blockIdx.x;
  const CJob& job = t.jobs[j];
  uint64_t c_lo = max(t.c_begin, job.chunk0);
  uint64_t c_hi = min(t.c_end, job.chunk0 + job.nchunks);
  if (job.nchunks == 0) {  // an empty tensor is only a header: the first group writes it
    if (t.c_begin != 0) return;
    c_lo = c_hi = job.chunk0;
  } else if (c_lo >= c_hi) {
    return;  // no chunk of this tensor in this launch
  }
  const bool first = c_lo == job.chunk0, final = c_hi == job.chunk0 + job.nchunks;
  // placement: the status of every chunk's top stream, its size when it
  // needs no coding (CONST, RAW), unknown (0) when k_encode codes it
  if (part == 1 && t.place) {
    for (uint64_t g = c_lo + threadIdx.x; g < c_hi; g += kScanThreads) {
      const uint64_t s = g * E + E - 1;
      const bool cand = (w.sinfo[4 * s + 1] & 0xFFu) == kModeCand;
      w.tstat[g] = cand ? 0ull : (g == job.chunk0 ? kStInc : kStAgg) | align16(w.sinfo[4 * s]);
    }
  }
  const uint64_t s0 = c_lo * E;
  // streams per chunk in this part, and the first of them
  const uint32_t per = part == 0 ? E : part == 1 ? E - 1 : 1u;
  const uint32_t k0 = part == 2 ? E - 1 : 0u;
  const uint64_t S = (c_hi - c_lo) * per;
  const uint64_t base = t.v2 ? w.pbase[j] : kHeader + kDirEntry * (uint64_t)job.nchunks * E;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  uint64_t running = part == 2 ? (first ? w.blob_nbytes[j] : w.top_run[j]) : first ? base : w.blob_nbytes[j];
  // global stream index of the idx-th stream of this part in the range
  auto sidx = [&](uint64_t idx) -> uint64_t {
    return per == E ? s0 + idx : s0 + (idx / per) * E + k0 + idx % per;
  };
  for (uint64_t tile = 0; tile < S; tile += 4 * kScanThreads) {
    uint64_t sz[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t idx = tile + 4 * tid + i;
      sz[i] = idx < S ? align16(w.sinfo[4 * sidx(idx)]) : 0;
      local += sz[i];
    }
    uint64_t inc = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t up = shfl_up_u64(inc, o);
      if (lane >= (uint32_t)o) inc += up;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint64_t before = 0, tile_total = 0;
    for (uint32_t q = 0; q < kScanThreads / 64; ++q) {
      if (q < wave) before += wave_tot[q];
      tile_total += wave_tot[q];
    }
    uint64_t off = running + before + inc - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t idx = tile + 4 * tid + i;
      if (idx < S) w.offsets[sidx(idx)] = off;
      off += sz[i];
    }
    running += tile_total;
    __syncthreads();
  }
  if (tid == 0) {
    if (part == 2) w.top_run[j] = running;
    else w.blob_nbytes[j] = running;
  }
  if (!final || part == 1) return;
  if (tid == 0) *job.blob_nbytes_out = running;
  if (tid < 4) {  // header
    uint4 v;
    if (tid == 0)
      v = make_uint4(0x4243544Cu /* "LTCB" */, (t.v2 ? 2u : 1u) | (t.dtype << 16) | (E << 24),
                     (uint32_t)job.nbytes, (uint32_t)(job.nbytes >> 32));
    else if (tid == 1)
      v = make_uint4(t.chunk_bytes, job.nchunks,
                     64u | (12u << 16) | ((t.v2 ? LTC_FLAG_SHARED_TABLES : 0u) << 24) |
                         ((t.delta ? LTC_FLAG_DELTA : 0u) << 24) | ((t.top_last ? LTC_FLAG_TOP_LAST : 0u) << 24),
                     0u);
    else if (tid == 2)
      v = make_uint4((uint32_t)running, (uint32_t)(running >> 32), (uint32_t)base,
                     (uint32_t)(base >> 32));
    else
      v = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(job.blob + 16 * tid) = v;
    if (t.crc) {
      // header unit tid sits at position tid of frame 0: its remainder
      // (bit by bit) times x^(8*16*(63 - tid)) is its share of the frame's
      uint32_t r = 0;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
      for (int q = 0; q < 4; ++q) {
        for (int b = 0; b < 4; ++b) {
          r ^= (wv[q] >> (8 * b)) & 0xFFu;
          for (int k = 0; k < 8; ++k) r = (r >> 1) ^ (kPoly & (0u - (r & 1u)));
        }
      }
      r = gf2_mulmod(r, t.crc_pos[tid]);
      if (r) atomicXor(job.frames, r);
    }
  }
}

// ------------------------------------------------------------------ k_pack

// 16 consecutive (reordered) elements of a chunk starting at element e0
// (zeros past n); deltas XOR the base in
template <int DT, bool DELTA = false>
__device__ __forceinline__ void load16(const uint8_t* src, uint32_t e0, uint32_t n, bool vec,
                                       uint32_t y[16], const uint8_t* bsrc = nullptr) {
  constexpr int E = Dt<DT>::E;
  if (vec && e0 + 16 <= n) {
    uint32_t wv[4 * E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
      const uint4 v = load_x16<DELTA>(src, bsrc, (uint64_t)e0 * E + 16 * q);
      wv[4 * q] = v.x;
      wv[4 * q + 1] = v.y;
      wv[4 * q + 2] = v.z;
      wv[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t x;
      if constexpr (E == 4) x = wv[i];
      else if constexpr (E == 2) x = (wv[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      else x = (wv[i / 4] >> (8 * (i & 3))) & 0xFFu;
      y[i] = reorder<DT>(x);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      y[i] = e0 + i < n ? reorder<DT>(load_x<DT, DELTA>(src, bsrc, (uint64_t)(e0 + i) * E)) : 0u;
  }
}

// ---- deltas: the zero-run coder's statistics and payload

// Zero-run statistics of a byte range: length, leading and trailing zero
// runs, longest zero run, all zero.  Ranges in order combine associatively.

// ZRUN payload of stream k of a chunk at dst (all threads of the workgroup;
// every byte of the payload and of its gap to 16 is written): 16-byte head,
// block bitmap (one ballot per 64 blocks), per nonzero block its byte mask at
// its rank, and the nonzero bytes at their rank.
template <int DT, bool DELTA>
__device__ void write_zrun(uint8_t* dst, const uint8_t* src, const uint8_t* bsrc, uint32_t n, int k,
                           uint32_t nblk, uint32_t nnz, uint32_t size, bool vec, uint32_t* red) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t nb = (n + 63) / 64;
  const uint32_t l1 = 16, l2 = l1 + (uint32_t)align16((nb + 7) / 8);
  const uint32_t lit = l2 + (uint32_t)align16(8ull * nblk);
  if (tid == 0) *reinterpret_cast<uint4*>(dst) = make_uint4(nnz, nblk, 0, 0);
  for (uint32_t i = l1 + 8 * ((nb + 63) / 64) + tid; i < l2; i += kPackThreads) dst[i] = 0;
  for (uint32_t i = l2 + 8 * nblk + tid; i < lit; i += kPackThreads) dst[i] = 0;
  for (uint32_t i = size + tid; i < align16(size); i += kPackThreads) dst[i] = 0;
  uint32_t run_blk = 0, run_lit = 0;
  for (uint32_t r0 = 0; r0 < nb; r0 += kPackThreads) {
    const uint32_t b = r0 + tid;
    uint64_t mask = 0;
    uint32_t by[16];  // the block's 64 stream bytes, 4 per word
#pragma unroll
    for (int i = 0; i < 16; ++i) by[i] = 0;
    if (b < nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t y[16];
        load16<DT, DELTA>(src, 64 * b + 16 * q, n, vec, y, bsrc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t v = (y[i] >> (8 * k)) & 0xFFu;
          by[4 * q + i / 4] |= v << (8 * (i & 3));
          if (v) mask |= 1ull << (16 * q + i);
        }
      }
    }
    const uint64_t bal = ballot(mask != 0);
    if (lane == 0 && r0 + 64 * wave < nb)
      *reinterpret_cast<uint64_t*>(dst + l1 + (r0 + 64 * wave) / 8) = bal;
    const uint32_t pc = (uint32_t)__popcll(mask);
    const uint32_t lit_below = wave_exclusive_scan_u32(pc);
    if (lane == 63) {
      red[wave] = (uint32_t)__popcll(bal);
      red[4 + wave] = lit_below + pc;
    }
    __syncthreads();
    uint32_t blk_before = run_blk, lit_before = run_lit, blk_round = 0, lit_round = 0;
    for (uint32_t q = 0; q < kPackThreads / 64; ++q) {
      if (q < wave) {
        blk_before += red[q];
        lit_before += red[4 + q];
      }
      blk_round += red[q];
      lit_round += red[4 + q];
    }
    __syncthreads();
    if (mask) {
      const uint32_t rank = lanes_below_plus(bal, blk_before);
      if (rank < nblk) *reinterpret_cast<uint64_t*>(dst + l2 + 8 * rank) = mask;
      uint32_t o = lit_before + lit_below;
      for (int i = 0; i < 64; ++i) {
        const uint32_t v = (by[i / 4] >> (8 * (i & 3))) & 0xFFu;
        if (v && o < nnz) dst[lit + o++] = (uint8_t)v;
      }
    }
    run_blk += blk_round;
    run_lit += lit_round;
  }
}

__device__ __forceinline__ uint32_t pack4(const uint32_t* y, int k) {
  return ((y[0] >> (8 * k)) & 0xFFu) | (((y[1] >> (8 * k)) & 0xFFu) << 8) |
         (((y[2] >> (8 * k)) & 0xFFu) << 16) | (((y[3] >> (8 * k)) & 0xFFu) << 24);
}

__device__ __forceinline__ uint32_t pack_u16x2(uint32_t a, uint32_t b) { return a | (b << 16); }

// ---- CRC-32 of the blob as it is written (compress_with_crc32)
// Blob bytes are checksummed in 16-byte units: a unit's remainder comes from
// slicing-by-8 tables, and the 64 units of a 1 KiB frame sit in the 64 lanes
// of a wave (lane = position in the frame).  A wave walks consecutive frames,
// so each lane first chains its units across frames (multiply by x^(8*1024)
// from byte tables, then add).  A run of frames ends at the last frame of a
// checksum chunk or of the wave's share; then each lane moves its chain to
// the end of the frame (times x^(8*16*(63 - lane)), bit by bit), the wave
// XORs the 64 values together, and lane 0 XORs the result, the run's
// remainder relative to the end of its last frame, into frames[last frame].
// Several workgroups can add to one frame where payloads meet; CRC linearity
// makes the XOR of the parts the remainder of the whole.

template <bool CRC> struct PackLds {};
template <> struct PackLds<true> { CrcLdsT<1> c; };  // t8 and x^(8*1024)

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o, 64);
  return v;
}

struct FrameRun {
  uint32_t acc;    // per lane
  uint64_t last;   // last frame added (uniform)
  uint32_t wpos;   // its position in its checksum chunk (uniform)
  bool open;
};

// pos: this lane's x^(8*16*(63 - lane)) mod P
__device__ __forceinline__ void run_flush(FrameRun& r, uint32_t pos, uint32_t* frames,
                                          uint32_t lane) {
  if (!r.open) return;
  const uint32_t v = wave_xor(gf2_mulmod(r.acc, pos));
  if (lane == 0 && v) atomicXor(frames + r.last, v);
  r.open = false;
}

// lanes hold unit remainders of 64 consecutive units starting at position
// rot of frame f: lanes below 64 - rot in frame f, the rest in frame f + 1
__device__ __forceinline__ void split_frames(uint32_t c, uint32_t rot, uint64_t f, uint32_t* frames,
                                             uint32_t pos, uint32_t lane) {
  const uint32_t v = __shfl(c, (lane - rot) & 63u, 64);  // lane = position in its frame
  const uint32_t m = gf2_mulmod(v, pos);
  const uint32_t lo = wave_xor(lane >= rot ? m : 0u), hi = wave_xor(lane < rot ? m : 0u);
  if (lane == 0) {
    if (lo) atomicXor(frames + f, lo);
    if (hi) atomicXor(frames + f + 1, hi);
  }
}

// lane l's unit remainder c at position l of frame f
__device__ __forceinline__ void run_add(FrameRun& r, const CrcLdsT<1>& s, uint32_t* frames,
                                        uint64_t f, uint32_t c, uint32_t per_chunk, uint32_t pos,
                                        uint32_t lane) {
  if (r.open && (f != r.last + 1 || r.wpos + 1 == per_chunk)) run_flush(r, pos, frames, lane);
  if (r.open) {
    r.acc = crc_mul_level(s, 0, r.acc) ^ c;
    r.wpos += 1;
  } else {
    r.acc = c;
    r.wpos = (uint32_t)(f % per_chunk);
    r.open = true;
  }
  r.last = f;
}

// frames [fb, fe) of a payload of `units` units starting at blob unit index a
// that this wave takes (contiguous shares, one per wave of the workgroup)
__device__ __forceinline__ void wave_frames(uint64_t a, uint32_t units, uint64_t& fb, uint64_t& fe) {
  constexpr uint64_t kWaves = kPackCrcThreads / 64;
  const uint64_t f0 = a >> 6, nf = ((a + units + 63) >> 6) - f0;
  const uint64_t q = (nf + kWaves - 1) / kWaves, wave = threadIdx.x / 64;
  fb = f0 + min(nf, wave * q);
  fe = f0 + min(nf, wave * q + q);
}

// unit u (16 bytes) of a RANS payload: prefix, states, frequencies, words
// y1: the prefix's second word (v1: sym_lo | sym_hi << 8; v2: 0); v2 payloads
// have no table (tcount 0, wo 272)
__device__ __forceinline__ uint4 rans_unit(uint32_t u, uint64_t s, uint32_t y1, uint32_t tcount,
                                           uint32_t wo, uint32_t nw, const uint16_t* fr,
                                           const uint16_t* words, const CWork& w) {
  const uint32_t pos = 16 * u;
  if (u == 0) return make_uint4(nw, y1, 0, 0);
  if (pos < kRansFixed) return *reinterpret_cast<const uint4*>(w.states + 64 * s + (pos - 16) / 4);
  uint32_t h[8];
  if (pos < wo) {
    const uint32_t i0 = (pos - kRansFixed) / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = i0 + i < tcount ? fr[i0 + i] : 0u;
  } else {
    const uint32_t i0 = (pos - wo) / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = i0 + i < nw ? words[i0 + i] : 0u;
  }
  return make_uint4(pack_u16x2(h[0], h[1]), pack_u16x2(h[2], h[3]), pack_u16x2(h[4], h[5]),
                    pack_u16x2(h[6], h[7]));
}

template <bool CRC>
__device__ void write_rans(uint8_t* blob, uint64_t off, uint64_t s, uint32_t info, uint32_t size,
                           uint32_t nw, const CTable& t, const CWork& w, uint32_t* frames,
                           const PackLds<CRC>& L, uint32_t pos) {
  const uint32_t lo = (info >> 16) & 0xFFu, hi = info >> 24;
  const uint32_t tcount = t.v2 ? 0u : hi - lo + 1u;
  const uint32_t wo = (uint32_t)align16(kRansFixed + 2u * tcount);
  const uint32_t y1 = t.v2 ? 0u : lo | (hi << 8);
  const uint32_t units = (uint32_t)(align16(size) / 16);
  const uint16_t* fr = w.freq + 256 * s + lo;
  const uint16_t* words = w.words + s * t.wcap + (t.wcap - nw);
  uint8_t* dst = blob + off;
  if constexpr (!CRC) {
    for (uint32_t u = threadIdx.x; u < units; u += kPackThreads)
      *reinterpret_cast<uint4*>(dst + 16 * u) = rans_unit(u, s, y1, tcount, wo, nw, fr, words, w);
  } else {
    const uint32_t lane = threadIdx.x & 63;
    const uint64_t a = off / 16;
    uint64_t fb, fe;
    wave_frames(a, units, fb, fe);
    FrameRun r{0, 0, 0, false};
    for (uint64_t f = fb; f < fe; ++f) {
      const uint64_t ua = 64 * f + lane;
      uint32_t c = 0;
      if (ua >= a && ua < a + units) {
        const uint32_t u = (uint32_t)(ua - a);
        const uint4 v = rans_unit(u, s, y1, tcount, wo, nw, fr, words, w);
        *reinterpret_cast<uint4*>(dst + 16 * u) = v;
        c = crc_step16(L.c, 0u, v);
      }
      run_add(r, L.c, frames, f, c, t.crc_frames, pos, lane);
    }
    run_flush(r, pos, frames, lane);
  }
}

template <int DT, bool CRC, bool DELTA>
__device__ __forceinline__ void pack_chunk(const CTable& t, const CWork& w, uint64_t g,
                                           const PackLds<CRC>& L, uint32_t pos, uint32_t* red) {
  constexpr int E = Dt<DT>::E;
  const int j = find_job(t, g);
  const CJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint8_t* src = job.src + c * t.chunk_bytes;
  uint8_t* blob = job.blob;
  const uint64_t s0 = g * E;
  const uint32_t tid = threadIdx.x;

  uint4 dir = make_uint4(0, 0, 0, 0);
  if (tid < (uint32_t)E) {
    const uint64_t s = s0 + tid;
    const uint4 si = *reinterpret_cast<const uint4*>(w.sinfo + 4 * s);
    const uint32_t mode = si.y & 0xFFu;
    const uint32_t cval = mode == LTC_MODE_CONST ? (si.y >> 8) & 0xFFu : 0u;
    const uint64_t off = w.offsets[s];
    dir = make_uint4((uint32_t)off, (uint32_t)(off >> 32), si.x, mode | (cval << 8));
    *reinterpret_cast<uint4*>(blob + kHeader + kDirEntry * (c * E + tid)) = dir;
  }
  if constexpr (CRC) {
    // the chunk's E directory entries: units 4 + c*E + k of the blob, in
    // lanes 0..E-1 of wave 0, rotated to their positions in their frame(s)
    if (tid < 64) {
      const uint32_t lane = tid;
      const uint32_t cr = lane < (uint32_t)E ? crc_step16(L.c, 0u, dir) : 0u;
      const uint64_t a = kHeader / 16 + c * E;
      split_frames(cr, (uint32_t)(a & 63), a >> 6, job.frames, pos, lane);
    }
  }
  // RAW streams: when k_encode staged them (stmask), already in place
  // (top-last layout, which the checksumming variant never packs: its
  // checksums are read back) or copied from their workspace slots; else
  // regrouped from the input
  uint32_t rawmask = 0, stmask = 0;
  uint64_t raw_off[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const uint64_t s = s0 + k;
    const uint4 si = *reinterpret_cast<const uint4*>(w.sinfo + 4 * s);
    const uint32_t mode = si.y & 0xFFu;
    raw_off[k] = w.offsets[s];
    if (mode == LTC_MODE_RAW) {
      rawmask |= 1u << k;
      if (si.w == kRawStaged) stmask |= 1u << k;
    }
    else if (mode == LTC_MODE_RANS && si.w != kPlaced)  // k_encode wrote the placed ones
      write_rans<CRC>(blob, raw_off[k], s, si.y, si.x, si.z, t, w, job.frames, L, pos);
    else if (DELTA && mode == LTC_MODE_ZRUN)
      write_zrun<DT, DELTA>(blob + raw_off[k], src, job.base + c * t.chunk_bytes, n, k, si.z, si.w, si.x,
                            t.vec16 != 0, red);
  }
  if (t.top_last) rawmask &= ~stmask;
  if (!rawmask) return;
  const uint32_t units = (n + 15) / 16;
  const bool regroup = (rawmask & ~stmask) != 0;
  // unit u of RAW stream k; y: the regrouped elements when not staged
  auto raw_unit = [&](int k, uint32_t u, const uint32_t* y) -> uint4 {
    if (stmask & (1u << k))
      return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(w.words + (s0 + k) * t.wcap) + 16 * u);
    return make_uint4(pack4(y, k), pack4(y + 4, k), pack4(y + 8, k), pack4(y + 12, k));
  };
  if constexpr (!CRC) {
    for (uint32_t u = tid; u < units; u += kPackThreads) {
      uint32_t y[16];
      if (regroup)
        load16<DT, DELTA>(src, 16 * u, n, t.vec16 != 0, y, DELTA ? job.base + c * t.chunk_bytes : nullptr);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (!(rawmask & (1u << k))) continue;
        *reinterpret_cast<uint4*>(blob + raw_off[k] + 16 * u) = raw_unit(k, u, y);
      }
    }
  } else {
    // frames follow the first RAW stream; another RAW stream at the same
    // position within its frames chains like it, one at another position
    // splits each wave's units over two frames (rotated, two trees per frame)
    const uint32_t lane = tid & 63;
    const int k0 = __builtin_ctz(rawmask);
    const uint64_t a0 = raw_off[k0] / 16;
    uint64_t fb, fe;
    wave_frames(a0, units, fb, fe);
    FrameRun r[E];
#pragma unroll
    for (int k = 0; k < E; ++k) r[k] = FrameRun{0, 0, 0, false};
    // With one or two streams, staged units load a frame ahead, so a load
    // is in flight while the current frame is checksummed (FP32's three
    // would not fit the 128 registers of 4 workgroups per CU).
    constexpr bool kAhead = E <= 2;
    uint4 nv[E];
    auto load_staged = [&](uint64_t f) {
      const uint64_t ua = 64 * f + lane;
      const bool have = ua >= a0 && ua < a0 + units;
#pragma unroll
      for (int k = 0; k < E; ++k)
        if (stmask & (1u << k)) nv[k] = have ? raw_unit(k, (uint32_t)(ua - a0), nullptr) : make_uint4(0, 0, 0, 0);
    };
    if (kAhead && fb < fe) load_staged(fb);
    for (uint64_t f = fb; f < fe; ++f) {
      const uint64_t ua = 64 * f + lane;
      const bool have = ua >= a0 && ua < a0 + units;
      const uint32_t u = (uint32_t)(ua - a0);
      uint4 cv[E];
      if constexpr (kAhead) {
#pragma unroll
        for (int k = 0; k < E; ++k) cv[k] = nv[k];
        if (f + 1 < fe) load_staged(f + 1);
      }
      uint32_t y[16];
      if (have && regroup) load16<DT>(src, 16 * u, n, t.vec16 != 0, y);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (!(rawmask & (1u << k))) continue;
        uint32_t cr = 0;
        if (have) {
          const uint4 v = (kAhead && (stmask & (1u << k))) ? cv[k] : raw_unit(k, u, y);
          *reinterpret_cast<uint4*>(blob + raw_off[k] + 16 * u) = v;
          cr = crc_step16(L.c, 0u, v);
        }
        const uint64_t d = raw_off[k] / 16 - a0;  // >= 0: streams are laid out in order
        const uint32_t rot = (uint32_t)(d & 63);
        const uint64_t fk = f + (d >> 6);
        if (rot == 0) run_add(r[k], L.c, job.frames, fk, cr, t.crc_frames, pos, lane);
        else split_frames(cr, rot, fk, job.frames, pos, lane);
      }
    }
#pragma unroll
    for (int k = 0; k < E; ++k) run_flush(r[k], pos, job.frames, lane);
  }
}

// One workgroup per chunk (a grid-stride loop).  The CRC variant builds its
// tables in every workgroup: measured no slower than a persistent grid of
// 1024 workgroups that builds them once each, and it lets checksummed calls
// use the pipelined groups.
template <int DT, bool CRC, bool DELTA>
__global__ __launch_bounds__(CRC ? kPackCrcThreads : kPackThreads)
__attribute__((amdgpu_waves_per_eu(CRC ? 4 : 1))) void k_pack(CTable t, CWork w) {
  __shared__ uint32_t red[8];  // ZRUN: per-wave counts
  __shared__ PackLds<CRC> lds;
  uint32_t pos = 0;
  if constexpr (CRC) {
    crc_build_tables(lds.c, &t.crc_x1k, threadIdx.x, kPackCrcThreads);
    pos = t.crc_pos[threadIdx.x & 63];
  }
  for (uint64_t g = t.c_begin + blockIdx.x; g < t.c_end; g += gridDim.x)
    pack_chunk<DT, CRC, DELTA>(t, w, g, lds, pos, red);
}

// ------------------------------------------------------------------ launch

// k_encode for stream indices kfirst, kfirst - 1, ... (nplanes of them) of
// chunks [t.c_begin, t.c_end), U streams per wave
template <int DT, bool DELTA, int U>
static void launch_encode_u(const CTable& t, const CWork& w, hipStream_t st, uint32_t kfirst,
                            uint32_t nplanes, uint64_t chunks) {
  const uint32_t grid = DELTA ? (uint32_t)((chunks + 8 * U - 1) / (8 * U) * 8 * nplanes)
                              : (uint32_t)((chunks + U - 1) / U * nplanes);
  hipLaunchKernelGGL((k_encode<DT, DELTA, 128, U>), dim3(grid), dim3(64), 0, st, t, w, kfirst, nplanes);
  hipLaunchKernelGGL((k_encode<DT, DELTA, 256, U>), dim3(grid), dim3(64), 0, st, t, w, kfirst, nplanes);
}

// Two interleaved streams per wave suit a call of many rounds of resident
// waves; a smaller call codes one stream per wave (54 instead of 101 VGPRs
// and half the LDS for BF16: 32 waves per CU instead of 16), so twice as many
// chains run at once and the last round is half as long.  Measured (top-last
// compress, one box): C2 (512 chunks) 0.154 -> 0.109 ms, C4b (1024) 0.291 ->
// 0.201 ms, C3 (13,312) 1.30 -> 1.27 ms; C5 (65,536) 5.45-5.49 ms with two
// streams against 5.59 with one.
constexpr uint64_t kEncPairMinChunks = 16384;

template <int DT, bool DELTA>
static void launch_encode(const CTable& t, const CWork& w, hipStream_t st, uint32_t kfirst,
                          uint32_t nplanes) {
  const uint64_t chunks = t.c_end - t.c_begin;
  if (!chunks || !nplanes) return;
  if (chunks < kEncPairMinChunks) launch_encode_u<DT, DELTA, 1>(t, w, st, kfirst, nplanes, chunks);
  else launch_encode_u<DT, DELTA, kEncStreams>(t, w, st, kfirst, nplanes, chunks);
}

template <int DT, bool DELTA>
static void launch_pack(const CTable& t, const CWork& w, hipStream_t st) {
  const uint64_t chunks = t.c_end - t.c_begin;
  if (!chunks) return;
  if constexpr (DELTA) {  // the blob is read back for checksums (no CRC variant)
    hipLaunchKernelGGL((k_pack<DT, false, true>), dim3((uint32_t)chunks), dim3(kPackThreads), 0, st, t, w);
  } else {
    if (t.crc)
      hipLaunchKernelGGL((k_pack<DT, true, false>), dim3((uint32_t)chunks), dim3(kPackCrcThreads), 0, st, t, w);
    else
      hipLaunchKernelGGL((k_pack<DT, false, false>), dim3((uint32_t)chunks), dim3(kPackThreads), 0, st, t, w);
  }
}

template <int DT, bool DELTA>
static hipError_t launch_compress_d(const CTable& t, const CWork& w, hipStream_t st,
                                    const hipEvent_t* ev, hipEvent_t scan_after,
                                    hipEvent_t scan_done, bool staged) {
  constexpr int E = Dt<DT>::E;
  const uint64_t chunks = t.c_end - t.c_begin;
  if (!staged) {
    record(ev, 0, st);
    if (chunks) hipLaunchKernelGGL((k_hist<DT, DELTA>), dim3((uint32_t)chunks), dim3(kHistThreads), 0, st, t, w);
    record(ev, 1, st);
  }
  launch_encode<DT, DELTA>(t, w, st, E - 1, E);
  record(ev, 2, st);
  if (scan_after) (void)hipStreamWaitEvent(st, scan_after, 0);
  hipLaunchKernelGGL(k_scan, dim3(t.count), dim3(kScanThreads), 0, st, t, w, (uint32_t)E, 0u);
  if (scan_done) (void)hipEventRecord(scan_done, st);
  record(ev, 3, st);
  launch_pack<DT, DELTA>(t, w, st);
  record(ev, 4, st);
  return hipGetLastError();
}

// Top-last layout, first half for chunks [c_begin, c_end): k_hist, the lower
// streams' coding, their scan, then the top streams' coding, which writes
// the staged RAW streams at the offsets that scan gave.  The profiling
// events put the lower streams' pass with k_hist, so that the second
// interval holds the top streams' coding alone.
template <int DT, bool DELTA>
static hipError_t launch_front_d(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                 hipEvent_t scan_after, hipEvent_t scan_done, bool staged) {
  constexpr int E = Dt<DT>::E;
  const uint64_t chunks = t.c_end - t.c_begin;
  if (!staged) {
    record(ev, 0, st);
    if (chunks) hipLaunchKernelGGL((k_hist<DT, DELTA>), dim3((uint32_t)chunks), dim3(kHistThreads), 0, st, t, w);
  }
  if (E > 1) launch_encode<DT, DELTA>(t, w, st, E - 2, E - 1);
  if (scan_after) (void)hipStreamWaitEvent(st, scan_after, 0);
  hipLaunchKernelGGL(k_scan, dim3(t.count), dim3(kScanThreads), 0, st, t, w, (uint32_t)E, 1u);
  if (scan_done) (void)hipEventRecord(scan_done, st);
  if (!staged) record(ev, 1, st);
  launch_encode<DT, DELTA>(t, w, st, E - 1, 1);
  record(ev, 2, st);
  return hipGetLastError();
}

// second half: the top streams' scan (the first group's needs every
// group's lower scan) and k_pack
template <int DT, bool DELTA>
static hipError_t launch_back_d(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                hipEvent_t scan_after, hipEvent_t scan_done) {
  constexpr int E = Dt<DT>::E;
  if (scan_after) (void)hipStreamWaitEvent(st, scan_after, 0);
  hipLaunchKernelGGL(k_scan, dim3(t.count), dim3(kScanThreads), 0, st, t, w, (uint32_t)E, 2u);
  if (scan_done) (void)hipEventRecord(scan_done, st);
  record(ev, 3, st);
  launch_pack<DT, DELTA>(t, w, st);
  record(ev, 4, st);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_compress_t(const CTable& t, const CWork& w, hipStream_t st,
                                    const hipEvent_t* ev, hipEvent_t scan_after,
                                    hipEvent_t scan_done, bool staged) {
  return t.delta ? launch_compress_d<DT, true>(t, w, st, ev, scan_after, scan_done, staged)
                 : launch_compress_d<DT, false>(t, w, st, ev, scan_after, scan_done, staged);
}

template <int DT>
static hipError_t launch_front_t(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                 hipEvent_t scan_after, hipEvent_t scan_done, bool staged) {
  return t.delta ? launch_front_d<DT, true>(t, w, st, ev, scan_after, scan_done, staged)
                 : launch_front_d<DT, false>(t, w, st, ev, scan_after, scan_done, staged);
}

template <int DT>
static hipError_t launch_back_t(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                hipEvent_t scan_after, hipEvent_t scan_done) {
  return t.delta ? launch_back_d<DT, true>(t, w, st, ev, scan_after, scan_done)
                 : launch_back_d<DT, false>(t, w, st, ev, scan_after, scan_done);
}

// v2, all chunks of t: histograms (summed per plane), plane tables and
// records, then the skip bound of every stream with its plane's table (and,
// for deltas, the zero-run statistics)
template <int DT>
static hipError_t launch_v2_tables_t(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev) {
  constexpr int E = Dt<DT>::E;
  const uint64_t chunks = t.c_end - t.c_begin;
  record(ev, 0, st);
  hipError_t err = launch_zero_u32(reinterpret_cast<uint32_t*>(w.plane), 2ull * 256 * E * t.count, st);
  if (err != hipSuccess) return err;
  if (chunks && t.delta)
    hipLaunchKernelGGL((k_hist<DT, true>), dim3((uint32_t)chunks), dim3(kHistThreads), 0, st, t, w);
  else if (chunks)
    hipLaunchKernelGGL((k_hist<DT, false>), dim3((uint32_t)chunks), dim3(kHistThreads), 0, st, t, w);
  if (chunks)
    hipLaunchKernelGGL(k_planesum<DT>, dim3((uint32_t)(E * ((chunks + kPlaneBlock - 1) / kPlaneBlock))),
                       dim3(256), 0, st, t, w);
  hipLaunchKernelGGL(k_share<DT>, dim3(t.count), dim3(256), 0, st, t, w);
  if (chunks) hipLaunchKernelGGL(k_decide<DT>, dim3((uint32_t)((chunks * E + 3) / 4)), dim3(256), 0, st, t, w);
  record(ev, 1, st);
  return hipGetLastError();
}

hipError_t launch_compress(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                           hipEvent_t scan_after, hipEvent_t scan_done, bool staged) {
  switch (t.dtype) {
    case LTC_U8: return launch_compress_t<LTC_U8>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_BF16: return launch_compress_t<LTC_BF16>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_FP16: return launch_compress_t<LTC_FP16>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_FP32: return launch_compress_t<LTC_FP32>(t, w, st, ev, scan_after, scan_done, staged);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_compress_front(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                 hipEvent_t scan_after, hipEvent_t scan_done, bool staged) {
  switch (t.dtype) {
    case LTC_U8: return launch_front_t<LTC_U8>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_BF16: return launch_front_t<LTC_BF16>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_FP16: return launch_front_t<LTC_FP16>(t, w, st, ev, scan_after, scan_done, staged);
    case LTC_FP32: return launch_front_t<LTC_FP32>(t, w, st, ev, scan_after, scan_done, staged);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_compress_back(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev,
                                hipEvent_t scan_after, hipEvent_t scan_done) {
  switch (t.dtype) {
    case LTC_U8: return launch_back_t<LTC_U8>(t, w, st, ev, scan_after, scan_done);
    case LTC_BF16: return launch_back_t<LTC_BF16>(t, w, st, ev, scan_after, scan_done);
    case LTC_FP16: return launch_back_t<LTC_FP16>(t, w, st, ev, scan_after, scan_done);
    case LTC_FP32: return launch_back_t<LTC_FP32>(t, w, st, ev, scan_after, scan_done);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_v2_tables(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev) {
  switch (t.dtype) {
    case LTC_U8: return launch_v2_tables_t<LTC_U8>(t, w, st, ev);
    case LTC_BF16: return launch_v2_tables_t<LTC_BF16>(t, w, st, ev);
    case LTC_FP16: return launch_v2_tables_t<LTC_FP16>(t, w, st, ev);
    case LTC_FP32: return launch_v2_tables_t<LTC_FP32>(t, w, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ltc
