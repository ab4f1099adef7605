// ltc_compress.hip -- gfx950 compression kernels.
//
// One compress call runs four kernels on the caller's stream:
//   k_hist    one workgroup per chunk: 16-byte loads, exponent-extracting
//             reorder, per-stream 256-bin histograms in LDS (lane-interleaved
//             sub-histograms against same-bin contention), then one wave per
//             stream normalises its histogram to a 4096 total and decides
//             CONST / RAW (by an exact lower bound on the rANS size) / encode.
//   k_encode  one wave per stream still to encode: 64-lane interleaved rANS
//             from the last step to the first, words staged in an LDS ring
//             and flushed 1 KiB at a time to the workspace; aborts to RAW as
//             soon as the payload can no longer beat the threshold.
//   k_scan    one workgroup per tensor: exclusive scan of the 16-byte-aligned
//             payload sizes into offsets; writes the 64-byte header.
//   k_pack    one workgroup per chunk: directory entries, RANS payloads from
//             the workspace, RAW streams regrouped from the input; every byte
//             of the blob, padding included, is written exactly once.
// Method: "NOTE-241: ZipNN", Method items 1-3 and 5; chunk size and
// passthrough rule: cuZipNN 0.1.0, API; interleaved rANS lanes and a table per
// stream: lmz README, "On a GPU" and "Building on lmz".
#include <type_traits>

#include "ltc_internal.h"
#include "ltc_launch.h"

namespace ltc {

constexpr int kHistThreads = 256;
constexpr int kHistCopies = 4;   // sub-histograms, picked by lane & 3
constexpr int kPackThreads = 256;
constexpr int kScanThreads = 1024;
constexpr uint32_t kRingWords = 1024;   // encoder word ring (LDS)
constexpr uint32_t kFlushWords = 512;   // one flush = 64 lanes x 16 bytes
constexpr int kEncBlock = 16;          // encoder steps per prefetched block

__device__ __forceinline__ uint32_t pack_info(uint32_t mode, uint32_t cval, uint32_t lo,
                                              uint32_t hi) {
  return mode | (cval << 8) | (lo << 16) | (hi << 24);
}

template <int DT> __device__ __forceinline__ uint32_t load_elem(const uint8_t* p) {
  constexpr int E = Dt<DT>::E;
  if constexpr (E == 1) return *p;
  else if constexpr (E == 2) return *reinterpret_cast<const uint16_t*>(p);
  else return *reinterpret_cast<const uint32_t*>(p);
}

// ------------------------------------------------------------------ k_hist

template <int DT>
__device__ __forceinline__ void hist_elem(uint32_t* hs, uint32_t y, uint32_t copy) {
  constexpr int E = Dt<DT>::E;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const uint32_t bin = (y >> (8 * k)) & 0xFFu;
    atomicAdd(&hs[(k * 256 + bin) * kHistCopies + copy], 1u);
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

// Normalise one stream's histogram (one wave; lane l owns symbols 4l..4l+3),
// pick CONST / RAW / encode, write the frequency table and the stream info.
__device__ void normalize_stream(const uint32_t* h, uint32_t n, uint32_t pmax, uint64_t s,
                                 const CWork& w) {
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
  if (nz == 1) {  // a single value: the stream is a header ("NOTE-241", Method item 3)
    if (lane == 0)
      *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = make_uint4(0, pack_info(LTC_MODE_CONST, lo, 0, 0), 0, 0);
    return;
  }
  uint32_t fsum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = hv[i] ? max(1u, (uint32_t)(((uint64_t)hv[i] << 12) / n)) : 0u;
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
    uint32_t key = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hv[i]) key = max(key, (hv[i] << 8) | (255u - (4 * lane + i)));
    key = wave_max_u32(key);
    const uint32_t v = 255u - (key & 255u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * lane + i == v) f[i] += kTotal - total;
  }
  // Lower bound on the rANS word count: each coding step gains at least
  // log2(4096/f) - log2(16/15) bits of state information (x >= 16 f there),
  // each renormalisation loses at most log2(16/15) (x >= 2^20 there), and the
  // 64 final states can hold at most 1024 bits more than the initial ones.
  // If even that bound exceeds P_max the stream is RAW whatever the encoder
  // would do, so it is not encoded.  64 bits of slack absorb rounding.
  double bits = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (hv[i]) bits += (double)hv[i] * (12.0 - log2((double)f[i]));
  bits = wave_sum_f64(bits);
  const uint32_t wo = (uint32_t)align16(kRansFixed + 2u * (hi - lo + 1u));
  const double wlb = (bits - 0.1862 * (double)n - 1024.0 - 64.0) / 16.0;
  const double plb = (double)wo + 2.0 * (wlb > 0.0 ? ceil(wlb) : 0.0);
  const bool raw = wo > pmax || plb > (double)pmax;
  const uint64_t packed = (uint64_t)f[0] | ((uint64_t)f[1] << 16) | ((uint64_t)f[2] << 32) |
                          ((uint64_t)f[3] << 48);
  *reinterpret_cast<uint64_t*>(w.freq + 256 * s + 4 * lane) = packed;
  if (lane == 0)
    *reinterpret_cast<uint4*>(w.sinfo + 4 * s) =
        make_uint4(raw ? n : 0u, pack_info(raw ? LTC_MODE_RAW : kModeCand, 0, lo, hi), 0, 0);
}

template <int DT>
__global__ __launch_bounds__(kHistThreads) void k_hist(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  __shared__ uint32_t hs[E * 256 * kHistCopies];
  __shared__ uint32_t hf[E * 256];
  const uint64_t g = blockIdx.x;
  const int j = find_job(t, g);
  const CJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint32_t len = n * E;
  const uint8_t* src = job.src + c * t.chunk_bytes;
  const uint32_t tid = threadIdx.x;
  const uint32_t copy = tid & (kHistCopies - 1);

  for (uint32_t i = tid; i < E * 256 * kHistCopies; i += kHistThreads) hs[i] = 0;
  __syncthreads();
  uint32_t done = 0;
  if (t.vec16 && len >= 16) {
    const uint32_t nvec = len / 16, lastv = nvec - 1;
    const uint4* v = reinterpret_cast<const uint4*>(src);
    // one 16-byte load in flight ahead of the one being counted; the index
    // is clamped instead of branched so the wait lands at the use
    uint4 q = v[min(tid, lastv)];
    for (uint32_t i = tid; i < nvec; i += kHistThreads) {
      const uint4 nq = v[min(i + kHistThreads, lastv)];
      hist_word<DT>(hs, q.x, copy);
      hist_word<DT>(hs, q.y, copy);
      hist_word<DT>(hs, q.z, copy);
      hist_word<DT>(hs, q.w, copy);
      q = nq;
    }
    done = nvec * 16;
  }
  for (uint32_t e = done / E + tid; e < n; e += kHistThreads)
    hist_elem<DT>(hs, reorder<DT>(load_elem<DT>(src + (uint64_t)e * E)), copy);
  __syncthreads();
  for (uint32_t i = tid; i < E * 256; i += kHistThreads) {
    uint32_t sum = 0;
#pragma unroll
    for (int r = 0; r < kHistCopies; ++r) sum += hs[i * kHistCopies + r];
    hf[i] = sum;
  }
  __syncthreads();
  const uint32_t wave = tid / 64;
  if (wave < (uint32_t)E)
    normalize_stream(hf + 256 * wave, n, last ? job.pmax_tail : job.pmax_full, g * E + wave, w);
}

// ---------------------------------------------------------------- k_encode

template <int DT>
__global__ __launch_bounds__(64) void k_encode(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  __shared__ uint4 tab[256];
  // word ring plus one private dummy slot per lane: a lane that emits
  // nothing writes its dummy slot, so the store needs no branch
  __shared__ __attribute__((aligned(16))) uint16_t ring[kRingWords + 64];
  const uint64_t s = blockIdx.x;
  const uint32_t info = w.sinfo[4 * s + 1];
  if ((info & 0xFFu) != kModeCand) return;
  const uint64_t g = s / E;
  const uint32_t k = (uint32_t)(s % E);
  const int j = find_job(t, g);
  const CJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint32_t pmax = last ? job.pmax_tail : job.pmax_full;
  const uint32_t lo = (info >> 16) & 0xFFu, hi = info >> 24;
  const uint32_t wo = (uint32_t)align16(kRansFixed + 2u * (hi - lo + 1u));
  const uint32_t lane = lane_id();

  // Encoder table, one 16-byte entry per symbol:
  //   x: f << 20, the renormalisation bound
  //   y: Granlund-Montgomery multiplier m for exact division by f
  //      (Granlund & Montgomery 1994, "Division by invariant integers using
  //      multiplication": q = (t + ((x - t) >> sh1)) >> sh2, t = mulhi(m, x))
  //   z: (4096 - f) | sh2 << 24   (the 24-bit multiply ignores the top byte)
  //   w: cum | sh1 << 24
  {
    const uint64_t fq = *reinterpret_cast<const uint64_t*>(w.freq + 256 * s + 4 * lane);
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
      const uint32_t fv = f[i];
      const uint32_t ell = fv <= 1 ? 0u : 32u - __clz(fv - 1u);
      const uint32_t m = fv ? (uint32_t)(((((uint64_t)1) << 32) * ((1ull << ell) - fv)) / fv + 1u) : 0u;
      const uint32_t sh1 = ell > 0 ? 1u : 0u, sh2 = ell > 0 ? ell - 1u : 0u;
      tab[4 * lane + i] = make_uint4(fv << 20, m, (kTotal - fv) | (sh2 << 24), (base + cum[i]) | (sh1 << 24));
    }
  }
  __syncthreads();

  const uint32_t wcap = t.wcap;
  uint16_t* wout = w.words + s * wcap;
  const uint32_t wlimit = (pmax - wo) / 2;  // more words than this cannot beat the threshold
  const uint8_t* src = job.src + c * t.chunk_bytes;
  const uint32_t full = n / 64;             // steps in which every lane codes a symbol
  const uint32_t steps = (n + 63) / 64;
  uint32_t x = kRansLow, top = wcap, nw = 0, flushed = 0;

  // Elements are fetched one block of steps ahead, unconditionally: lanes
  // past the end read the last element instead (their state is not
  // updated), so no branch forces an early wait on the loads.
  auto elem_at = [&](uint32_t step) -> uint32_t {
    const uint32_t e = 64 * step + lane;
    return load_elem<DT>(src + (uint64_t)(e < n ? e : n - 1) * E);
  };
  auto flush = [&](uint32_t b) {
    __syncthreads();
    const uint32_t base = wcap - kFlushWords * (b + 1) + 8 * lane;
    const uint4 v = *reinterpret_cast<const uint4*>(&ring[base & (kRingWords - 1)]);
    *reinterpret_cast<uint4*>(wout + base) = v;
  };
  // One coding step of the wave.  Steps run from the last to the first and,
  // within a step, the emitted words take decoder order (lanes ascending):
  // lane l's word goes to top - cnt + (number of emitting lanes below l).
  // Returns false once the payload can no longer beat the threshold.
  auto code = [&](auto guarded, uint32_t raw) -> bool {
    constexpr bool G = decltype(guarded)::value;
    const bool active = !G || 64 * full + lane < n;
    const uint4 e = tab[(reorder<DT>(raw) >> (8 * k)) & 0xFFu];
    const bool need = active && x >= e.x;
    const uint64_t mask = ballot(need);
    const uint32_t cnt = (uint32_t)__popcll(mask);
    nw += cnt;
    if (nw > wlimit) return false;
    const uint32_t slot = need ? ((top - cnt + lanes_below(mask)) & (kRingWords - 1)) : kRingWords + lane;
    ring[slot] = (uint16_t)x;
    const uint32_t xr = need ? x >> 16 : x;
    top -= cnt;
    const uint32_t t1 = __umulhi(e.y, xr);
    const uint32_t q = (t1 + ((xr - t1) >> (e.w >> 24))) >> (e.z >> 24);
    const uint32_t xn = __umul24(q, e.z) + xr + (e.w & 0xFFFFFFu);
    x = active ? xn : x;
    if (nw >= kFlushWords * (flushed + 1)) {
      flush(flushed);
      ++flushed;
    }
    return true;
  };

  bool ok = true;
  if (steps > full) ok = code(std::true_type{}, elem_at(full));  // the partial step comes first
  if (ok && full > 0) {
    const uint32_t nblk = (full + kEncBlock - 1) / kEncBlock;
    uint32_t cur[kEncBlock];
#pragma unroll
    for (int q = 0; q < kEncBlock; ++q) cur[q] = elem_at(kEncBlock * (nblk - 1) + q);
    for (int b = (int)nblk - 1; b >= 0 && ok; --b) {
      uint32_t nxt[kEncBlock];
#pragma unroll
      for (int q = 0; q < kEncBlock; ++q) nxt[q] = elem_at(kEncBlock * (b > 0 ? b - 1 : 0) + q);
#pragma unroll
      for (int q = kEncBlock - 1; q >= 0; --q) {
        if (kEncBlock * (uint32_t)b + q >= full) continue;
        if (!code(std::false_type{}, cur[q])) {
          ok = false;
          break;
        }
      }
#pragma unroll
      for (int q = 0; q < kEncBlock; ++q) cur[q] = nxt[q];
    }
  }
  if (!ok) {
    if (lane == 0)
      *reinterpret_cast<uint4*>(w.sinfo + 4 * s) = make_uint4(n, pack_info(LTC_MODE_RAW, 0, 0, 0), 0, 0);
    return;
  }
  if (nw > kFlushWords * flushed) flush(flushed);
  w.states[64 * s + lane] = x;
  if (lane == 0)
    *reinterpret_cast<uint4*>(w.sinfo + 4 * s) =
        make_uint4(wo + 2 * nw, pack_info(LTC_MODE_RANS, 0, lo, hi), nw, 0);
}

// ------------------------------------------------------------------ k_scan

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_up((uint32_t)v, o, 64);
  const uint32_t hi = __shfl_up((uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

__global__ __launch_bounds__(kScanThreads) void k_scan(CTable t, CWork w, uint32_t E) {
  __shared__ uint64_t wave_tot[kScanThreads / 64];
  const int j = blockIdx.x;
  const CJob& job = t.jobs[j];
  const uint64_t s0 = job.chunk0 * E;
  const uint64_t S = (uint64_t)job.nchunks * E;
  const uint64_t base = kHeader + kDirEntry * S;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  uint64_t running = base;
  for (uint64_t tile = 0; tile < S; tile += 4 * kScanThreads) {
    uint64_t sz[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint64_t idx = tile + 4 * tid + i;
      sz[i] = idx < S ? align16(w.sinfo[4 * (s0 + idx)]) : 0;
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
      if (idx < S) w.offsets[s0 + idx] = off;
      off += sz[i];
    }
    running += tile_total;
    __syncthreads();
  }
  if (tid == 0) {
    w.blob_nbytes[j] = running;
    *job.blob_nbytes_out = running;
  }
  if (tid < 4) {  // header
    uint4 v;
    if (tid == 0)
      v = make_uint4(0x4243544Cu /* "LTCB" */, 1u | (t.dtype << 16) | (E << 24),
                     (uint32_t)job.nbytes, (uint32_t)(job.nbytes >> 32));
    else if (tid == 1)
      v = make_uint4(t.chunk_bytes, job.nchunks, 64u | (12u << 16), 0u);
    else if (tid == 2)
      v = make_uint4((uint32_t)running, (uint32_t)(running >> 32), (uint32_t)base,
                     (uint32_t)(base >> 32));
    else
      v = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(job.blob + 16 * tid) = v;
  }
}

// ------------------------------------------------------------------ k_pack

// 16 consecutive elements of a chunk starting at element e0 (zeros past n)
template <int DT>
__device__ __forceinline__ void load16(const uint8_t* src, uint32_t e0, uint32_t n, bool vec,
                                       uint32_t y[16]) {
  constexpr int E = Dt<DT>::E;
  if (vec && e0 + 16 <= n) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (uint64_t)e0 * E);
    uint32_t wv[4 * E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
      const uint4 v = p[q];
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
      y[i] = e0 + i < n ? reorder<DT>(load_elem<DT>(src + (uint64_t)(e0 + i) * E)) : 0u;
  }
}

__device__ __forceinline__ uint32_t pack4(const uint32_t* y, int k) {
  return ((y[0] >> (8 * k)) & 0xFFu) | (((y[1] >> (8 * k)) & 0xFFu) << 8) |
         (((y[2] >> (8 * k)) & 0xFFu) << 16) | (((y[3] >> (8 * k)) & 0xFFu) << 24);
}

__device__ __forceinline__ uint32_t pack_u16x2(uint32_t a, uint32_t b) { return a | (b << 16); }

__device__ void write_rans(uint8_t* dst, uint64_t s, uint32_t info, uint32_t size, uint32_t nw,
                           const CTable& t, const CWork& w) {
  const uint32_t lo = (info >> 16) & 0xFFu, hi = info >> 24;
  const uint32_t tcount = hi - lo + 1u;
  const uint32_t wo = (uint32_t)align16(kRansFixed + 2u * tcount);
  const uint32_t units = (uint32_t)(align16(size) / 16);
  const uint16_t* fr = w.freq + 256 * s + lo;
  const uint16_t* words = w.words + s * t.wcap + (t.wcap - nw);
  for (uint32_t u = threadIdx.x; u < units; u += kPackThreads) {
    const uint32_t pos = 16 * u;
    uint4 v;
    if (u == 0) {
      v = make_uint4(nw, lo | (hi << 8), 0, 0);
    } else if (pos < kRansFixed) {
      v = *reinterpret_cast<const uint4*>(w.states + 64 * s + (pos - 16) / 4);
    } else {
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
      v = make_uint4(pack_u16x2(h[0], h[1]), pack_u16x2(h[2], h[3]), pack_u16x2(h[4], h[5]),
                     pack_u16x2(h[6], h[7]));
    }
    *reinterpret_cast<uint4*>(dst + pos) = v;
  }
}

template <int DT>
__global__ __launch_bounds__(kPackThreads) void k_pack(CTable t, CWork w) {
  constexpr int E = Dt<DT>::E;
  const uint64_t g = blockIdx.x;
  const int j = find_job(t, g);
  const CJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint8_t* src = job.src + c * t.chunk_bytes;
  uint8_t* blob = job.blob;
  const uint64_t s0 = g * E;
  const uint32_t tid = threadIdx.x;

  if (tid < (uint32_t)E) {
    const uint64_t s = s0 + tid;
    const uint4 si = *reinterpret_cast<const uint4*>(w.sinfo + 4 * s);
    const uint32_t mode = si.y & 0xFFu;
    const uint32_t cval = mode == LTC_MODE_CONST ? (si.y >> 8) & 0xFFu : 0u;
    const uint64_t off = w.offsets[s];
    *reinterpret_cast<uint4*>(blob + kHeader + kDirEntry * (c * E + tid)) =
        make_uint4((uint32_t)off, (uint32_t)(off >> 32), si.x, mode | (cval << 8));
  }
  uint32_t rawmask = 0;
  uint64_t raw_off[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const uint64_t s = s0 + k;
    const uint4 si = *reinterpret_cast<const uint4*>(w.sinfo + 4 * s);
    const uint32_t mode = si.y & 0xFFu;
    raw_off[k] = w.offsets[s];
    if (mode == LTC_MODE_RAW) rawmask |= 1u << k;
    else if (mode == LTC_MODE_RANS) write_rans(blob + raw_off[k], s, si.y, si.x, si.z, t, w);
  }
  if (rawmask) {
    const uint32_t units = (n + 15) / 16;
    for (uint32_t u = tid; u < units; u += kPackThreads) {
      uint32_t y[16];
      load16<DT>(src, 16 * u, n, t.vec16 != 0, y);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (!(rawmask & (1u << k))) continue;
        const uint4 v = make_uint4(pack4(y, k), pack4(y + 4, k), pack4(y + 8, k), pack4(y + 12, k));
        *reinterpret_cast<uint4*>(blob + raw_off[k] + 16 * u) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ launch

template <int DT>
static hipError_t launch_compress_t(const CTable& t, const CWork& w, hipStream_t st,
                                    const hipEvent_t* ev) {
  constexpr int E = Dt<DT>::E;
  const uint64_t chunks = t.total_chunks;
  record(ev, 0, st);
  if (chunks) hipLaunchKernelGGL(k_hist<DT>, dim3((uint32_t)chunks), dim3(kHistThreads), 0, st, t, w);
  record(ev, 1, st);
  if (chunks) hipLaunchKernelGGL(k_encode<DT>, dim3((uint32_t)(chunks * E)), dim3(64), 0, st, t, w);
  record(ev, 2, st);
  hipLaunchKernelGGL(k_scan, dim3(t.count), dim3(kScanThreads), 0, st, t, w, (uint32_t)E);
  record(ev, 3, st);
  if (chunks) hipLaunchKernelGGL(k_pack<DT>, dim3((uint32_t)chunks), dim3(kPackThreads), 0, st, t, w);
  record(ev, 4, st);
  return hipGetLastError();
}

hipError_t launch_compress(const CTable& t, const CWork& w, hipStream_t st, const hipEvent_t* ev) {
  switch (t.dtype) {
    case LTC_U8: return launch_compress_t<LTC_U8>(t, w, st, ev);
    case LTC_BF16: return launch_compress_t<LTC_BF16>(t, w, st, ev);
    case LTC_FP16: return launch_compress_t<LTC_FP16>(t, w, st, ev);
    case LTC_FP32: return launch_compress_t<LTC_FP32>(t, w, st, ev);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ltc
