// ltc_decompress.hip -- gfx950 decoding kernel.
//
// One wave64 workgroup per chunk.  The 64 interleaved rANS lanes of a coded
// stream are the 64 lanes of the wave (lmz README, "On a GPU": the
// interleaved states are the lanes of work, so parallelism comes from many
// streams at once).  Per chunk the wave
//   1. checks its directory entries (offset chain, modes, sizes) and the
//      RANS payload headers (symbol range, zero fields, table sum, states),
//   2. builds, per coded stream, a 4096-slot symbol table (u8) and a
//      per-symbol (f, cum) table in LDS,
//   3. streams the coded words through a 1024-word LDS ring of four
//      256-word slots, refilled once per block from registers loaded a
//      retirement ahead,
//   4. decodes 8 steps (512 symbols) at a time, writing the symbols in
//      element order into the ring's dead slot,
//   5. rebuilds the elements from those symbols (coded streams), direct
//      loads (RAW streams) and constants (CONST streams), undoes the exponent
//      extraction and writes 8 elements per lane with one vector store.
// The decoding loop is a dependent chain (table lookup -> state update ->
// conditional word fetch), which lmz's README calls latency-bound; many
// resident waves hide it.  The full blocks of a chunk with one coded stream
// run in a loop whose memory operations come in a fixed order, so that no
// wait for a load also waits for the output stores (see the fast loop).
// Chunks with more than one coded stream go to a second instantiation that
// holds several tables.
#include <type_traits>

#include "ltc_internal.h"
#include "ltc_launch.h"

namespace ltc {

constexpr uint32_t kDecRing = 1024;  // words: four slots of 256
constexpr uint32_t kMirror = 64;     // words after the ring: a copy of its first 64
// chunks (one wave each, independent) per workgroup.  Measured on 13,312
// BF16 chunks: 1 -> 0.720-0.727 ms, 2 -> 0.729-0.732 ms, 4 -> 0.735-0.740 ms
// (fewer workgroups to dispatch, but each holds its CU slot until its
// slowest chunk ends).
constexpr uint32_t kDecWaves = 1;
constexpr uint32_t kHalf = 256;     // words per refill (64 lanes x 8 bytes)
// Launches of at most this many chunks decode with the fused slot table
// (8 waves per CU: every chunk of such a launch is resident at once).
constexpr uint64_t kDecFusedMaxChunks = 2048;

// Words 256h + 4l .. +3 of a coded stream (lane l).  An 8-byte read that
// starts at a word index below W stays inside the payload's 16-byte padded
// slot, so only the start index is clamped (no branch, no early wait); a
// stream with W = 0 passes a pointer into the directory instead.  Words past
// W are never consumed by a valid blob, and reading one marks it corrupt.
__device__ __forceinline__ uint2 load_half(const uint16_t* wp, uint32_t nw, uint32_t h) {
  const uint32_t idx = kHalf * h + 4 * lane_id();
  return *reinterpret_cast<const uint2*>(wp + (idx < nw ? idx : 0u));
}

// 8 bytes of a RAW stream at element e0; the 16-byte padding of the payload
// slot covers a read that starts below n, lanes past the end read offset 0.
__device__ __forceinline__ uint64_t load_raw8(const uint8_t* rp, uint32_t e0, uint32_t n) {
  return *reinterpret_cast<const uint64_t*>(rp + (e0 < n ? e0 : 0u));
}

__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t a, uint32_t b) {
  return (a & mask) | (b & ~mask);  // v_bfi_b32
}

// Four elements from their E stream bytes (one 32-bit word per stream, byte
// i belongs to element i): undoes the byte grouping and the exponent
// extraction with bit inserts and byte permutes on packed bytes.
template <int DT> __device__ __forceinline__ void planes_to_words(const uint32_t* p, uint32_t* o) {
  if constexpr (DT == LTC_U8) {
    o[0] = p[0];
  } else if constexpr (DT == LTC_BF16) {
    // stream 1 = e, stream 0 = s<<7 | m; element = s<<15 | e<<7 | m
    const uint32_t hi = bit_insert(0x80808080u, p[0], p[1] >> 1);  // s<<7 | e>>1
    const uint32_t lo = bit_insert(0x80808080u, p[1] << 7, p[0]);  // (e&1)<<7 | m
    o[0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    o[1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  } else if constexpr (DT == LTC_FP16) {
    // stream 1 = e<<3 | s<<2 | m[9:8]; high byte = s<<7 | e<<2 | m[9:8]
    const uint32_t hi = bit_insert(0x80808080u, p[1] << 5, bit_insert(0x7C7C7C7Cu, p[1] >> 1, p[1]));
    o[0] = __builtin_amdgcn_perm(hi, p[0], 0x05010400u);
    o[1] = __builtin_amdgcn_perm(hi, p[0], 0x07030602u);
  } else {
    // stream 3 = e, stream 2 = s<<7 | m[22:16], streams 1, 0 = m[15:8], m[7:0]
    const uint32_t b3 = bit_insert(0x80808080u, p[2], p[3] >> 1);
    const uint32_t b2 = bit_insert(0x80808080u, p[3] << 7, p[2]);
    const uint32_t a = __builtin_amdgcn_perm(p[1], p[0], 0x05010400u);
    const uint32_t b = __builtin_amdgcn_perm(p[1], p[0], 0x07030602u);
    const uint32_t c = __builtin_amdgcn_perm(b3, b2, 0x05010400u);
    const uint32_t d = __builtin_amdgcn_perm(b3, b2, 0x07030602u);
    o[0] = __builtin_amdgcn_perm(c, a, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(c, a, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(d, b, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(d, b, 0x07060302u);
  }
}

// FUSED (one coded stream per chunk, small calls): one 32-bit entry per slot,
// symbol | f << 8 | (slot - cum) << 20 (a coded stream has two or more
// symbols, so f and slot - cum stay below 4096), read once per step instead
// of the slot's symbol and then the symbol's (f, cum).  The 16 KiB table
// leaves room for 8 waves per CU instead of 20, which a call of at most
// kDecFusedMaxChunks chunks does not fill anyway.
template <int DT, int MAXR, bool DELTA, bool FUSED = false>
__global__ __launch_bounds__(64 * kDecWaves) void k_decode(DTable t) {
  constexpr int E = Dt<DT>::E;
  static_assert(!FUSED || MAXR == 1, "the fused table serves one coded stream");
  __shared__ uint8_t lut_w[kDecWaves][MAXR][FUSED ? 4 : 4096];
  __shared__ uint32_t symt_w[kDecWaves][MAXR][FUSED ? 4096 : 256];
  __shared__ __attribute__((aligned(16))) uint16_t ring_w[kDecWaves][MAXR][kDecRing + kMirror];
  const uint32_t wslot = kDecWaves > 1 ? threadIdx.x / 64 : 0u;
  auto& lut = lut_w[wslot];
  auto& symt = symt_w[wslot];
  auto& ring = ring_w[wslot];

  const uint64_t g = t.c_begin + (uint64_t)blockIdx.x * kDecWaves + wslot;
  if (g >= t.c_end) return;
  const int j = find_job(t, g);
  const DJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const bool last = c + 1 == job.nchunks;
  const uint32_t n = last ? job.n_tail : t.n_full;
  const uint8_t* blob = job.blob;
  const uint64_t B = job.blob_nbytes;
  const uint64_t S = (uint64_t)job.nchunks * E;
  const uint64_t s0 = c * E;
  const uint32_t lane = lane_id();

  // ---- directory
  const uint4* dir = reinterpret_cast<const uint4*>(blob + kHeader);
  uint64_t off[E];
  uint32_t size[E], mode[E], cval[E];
  bool bad = false;
  int nr = 0;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const uint4 e = dir[s0 + k];
    off[k] = (uint64_t)e.x | ((uint64_t)e.y << 32);
    size[k] = e.z;
    mode[k] = e.w & 0xFFu;
    cval[k] = (e.w >> 8) & 0xFFu;
    bad |= (e.w >> 16) != 0 || mode[k] > (DELTA ? 3u : 2u) || (mode[k] != LTC_MODE_CONST && cval[k] != 0) ||
           (mode[k] == LTC_MODE_ZRUN && size[k] < 16) ||
           (mode[k] == LTC_MODE_RAW && size[k] != n) || (mode[k] == LTC_MODE_CONST && size[k] != 0) ||
           (mode[k] == LTC_MODE_RANS && size[k] < kRansFixed + (job.v2 ? 0u : 16u)) || off[k] > B ||
           (uint64_t)size[k] > B - off[k];
    nr += mode[k] == LTC_MODE_RANS;
  }
  // the offset chain: every payload starts where the one before it in blob
  // order ends, rounded up to 16; the first at payload_base, the last ends
  // the blob.  Directory order: the chunk's own links and the link to the
  // next chunk.  Top-last: the link into each of the chunk's streams.
  if (E > 1 && job.top_last) {
    auto end_of = [&](uint64_t si) -> uint64_t {  // where entry si's payload ends
      const uint4 e = dir[si];
      return align16(((uint64_t)e.x | ((uint64_t)e.y << 32)) + e.z);
    };
    bad |= off[0] != (c == 0 ? job.payload_base : end_of(s0 - 2));  // after stream E-2 of chunk c-1
#pragma unroll
    for (int k = 1; k < E - 1; ++k) bad |= off[k] != align16(off[k - 1] + size[k - 1]);
    // after the last lower stream of the blob, or the top stream of chunk c-1
    bad |= off[E - 1] != (c == 0 ? end_of(S - 2) : end_of(s0 - 1));
    if (last) bad |= align16(off[E - 1] + size[E - 1]) != B;
  } else {
    if (c == 0) bad |= off[0] != job.payload_base;
#pragma unroll
    for (int k = 1; k < E; ++k) bad |= off[k] != align16(off[k - 1] + size[k - 1]);
    const uint64_t end = align16(off[E - 1] + size[E - 1]);
    if (s0 + E < S) {
      const uint4 e = dir[s0 + E];
      bad |= ((uint64_t)e.x | ((uint64_t)e.y << 32)) != end;
    } else {
      bad |= end != B;
    }
  }
  if (MAXR == 1) {
    if (bad) {
      if (lane == 0) *job.status = LTC_ERR_CORRUPT;
      return;
    }
    if (nr > 1) return;  // the multi-table instantiation takes it
  } else if (bad || nr <= 1) {
    return;
  }

  // ---- v2: the table records between the directory and payload_base (each
  // chunk finds its planes' records; chunk 0 also checks every table, so the
  // verdict on a blob does not depend on which planes are used)
  const uint8_t* recs[E];
  uint32_t rlo[E], rhi[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    recs[k] = nullptr;
    rlo[k] = 1;
    rhi[k] = 0;
  }
  if (job.v2) {
    const uint8_t* cur = blob + kHeader + kDirEntry * S;
    const uint8_t* end = blob + job.payload_base;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      if (bad || cur + 16 > end) {
        bad = true;
        break;
      }
      const uint4 h = *reinterpret_cast<const uint4*>(cur);
      const uint32_t lo = h.x & 0xFFFFu, hi = h.x >> 16;
      const bool absent = lo == 1 && hi == 0;
      bad |= h.y != 0 || h.z != 0 || h.w != 0 || (!absent && (lo >= hi || hi > 255));
      if (bad) break;
      recs[k] = cur;
      rlo[k] = lo;
      rhi[k] = hi;
      cur += absent ? 16u : (uint32_t)align16(16u + 2u * (hi - lo + 1u));
    }
    bad |= cur != end;
    if (c == 0 && !bad) {
#pragma unroll
      for (int k = 0; k < E; ++k) {
        if (rlo[k] > rhi[k]) continue;
        const uint32_t tcount = rhi[k] - rlo[k] + 1u;
        const uint16_t* ft = reinterpret_cast<const uint16_t*>(recs[k] + 16);
        uint32_t acc = 0, flast = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t i = 4 * lane + q;
          const uint32_t fv = i < tcount ? ft[i] : 0u;
          acc += fv;
          if (i == tcount - 1) flast = fv;
        }
        const uint32_t pad = (uint32_t)align16(2u * tcount) - 2u * tcount;
        const bool padbad = lane < pad && recs[k][16 + 2 * tcount + lane] != 0;
        bad |= wave_sum_u32(acc) != kTotal || __shfl(ft[0], 0, 64) == 0 || wave_max_u32(flast) == 0 ||
               ballot(padbad) != 0;
      }
    }
    if (bad) {  // exactly one of the two instantiations gets here for a chunk
      if (lane == 0) *job.status = LTC_ERR_CORRUPT;
      return;
    }
  }

  // ---- coded-stream headers and tables
  int rstream[MAXR];
  uint32_t tlo[MAXR], tcnt[MAXR];
  uint32_t x[MAXR], nwords[MAXR], pos[MAXR], hcur[MAXR];
  uint2 staged[MAXR];
  const uint16_t* wp[MAXR];
  int slot_of[E];
  {
    int rr = 0;
#pragma unroll
    for (int k = 0; k < E; ++k) {
      slot_of[k] = -1;
      if (mode[k] == LTC_MODE_RANS && rr < MAXR) {
        slot_of[k] = rr;
        rstream[rr] = k;
        ++rr;
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    x[rr] = kRansLow;
    nwords[rr] = 0;
    pos[rr] = 0;
    hcur[rr] = 0;
    wp[rr] = nullptr;
    tlo[rr] = 0;
    tcnt[rr] = 0;
    if (rr >= nr) continue;
    const int k = rstream[rr];
    const uint8_t* p = blob + off[k];
    const uint4 h = *reinterpret_cast<const uint4*>(p);
    // the table (u16 f[lo..hi] then zero pad to 16): v1 in the payload after
    // the states, v2 in the plane's record
    uint32_t lo, hi, wo;
    const uint8_t* tb;
    if (job.v2) {
      lo = rlo[k];
      hi = rhi[k];
      wo = kRansFixed;
      tb = recs[k] + 16;
      bad |= lo >= hi || h.y != 0 || h.z != 0 || h.w != 0 || (uint64_t)(size[k] - wo) != 2ull * h.x;
    } else {
      lo = h.y & 0xFFu;
      hi = (h.y >> 8) & 0xFFu;
      wo = (uint32_t)align16(kRansFixed + 2u * (hi - lo + 1u));
      tb = p + kRansFixed;
      bad |= lo >= hi || (h.y >> 16) != 0 || h.z != 0 || h.w != 0 || wo > size[k] ||
             (uint64_t)(size[k] - wo) != 2ull * h.x;
    }
    if (bad) break;
    const uint32_t tcount = hi - lo + 1u;
    tlo[rr] = lo;
    tcnt[rr] = tcount;
    nwords[rr] = h.x;
    // with no words, refills (reached only by a corrupt stream) read the
    // directory, which is always inside the blob
    wp[rr] = reinterpret_cast<const uint16_t*>(h.x ? p + wo : blob + kHeader);
    x[rr] = reinterpret_cast<const uint32_t*>(p + 16)[lane];
    bad |= ballot(x[rr] < kRansLow) != 0;
    const uint16_t* ft = reinterpret_cast<const uint16_t*>(tb);
    uint32_t f[4], cum[4], acc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t i = 4 * lane + q;
      f[q] = i < tcount ? ft[i] : 0u;
      cum[q] = acc;
      acc += f[q];
    }
    const uint32_t base = wave_exclusive_scan_u32(acc);
    const uint32_t total = wave_sum_u32(acc);
    uint32_t flast = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * lane + q == tcount - 1) flast = f[q];
    const uint32_t f_lo = __shfl(f[0], 0, 64);
    const uint32_t f_hi = wave_max_u32(flast);
    const uint32_t pad = (uint32_t)align16(2u * tcount) - 2u * tcount;
    const bool padbad = lane < pad && tb[2 * tcount + lane] != 0;
    bad |= total != kTotal || f_lo == 0 || f_hi == 0 || ballot(padbad) != 0;
    if (bad) break;
    uint16_t* cumt = ring[rr];  // the ring doubles as the cum table while building
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t i = 4 * lane + q;
      if (i < tcount) {
        if constexpr (!FUSED) symt[rr][lo + i] = f[q] | ((base + cum[q]) << 16);
        cumt[i] = (uint16_t)(base + cum[q]);
      }
    }
    if (lane == 0) cumt[tcount] = (uint16_t)kTotal;
  }
  if (bad) {
    if (lane == 0) *job.status = LTC_ERR_CORRUPT;
    return;
  }
  wave_sync();
  // slot -> symbol table: lane l fills slots 64l .. 64l+63 (FUSED: the slot
  // entries, lane l slots l, l + 64, ..., so that consecutive lanes write
  // consecutive words)
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    if (rr >= nr) continue;
    const uint32_t lo = tlo[rr], tcount = tcnt[rr];
    const uint16_t* cumt = ring[rr];
    if constexpr (FUSED) {
      uint32_t a = 0, z = tcount - 1;  // largest i with cumt[i] <= lane
      while (a < z) {
        const uint32_t mid = (a + z + 1) / 2;
        if (cumt[mid] <= lane) a = mid;
        else z = mid - 1;
      }
      uint32_t v = a, curc = cumt[a], nextc = cumt[a + 1];  // cumt[tcount] = 4096 ends every walk
      for (uint32_t j = 0; j < 64; ++j) {
        const uint32_t sl = lane + 64 * j;
        while (nextc <= sl) {
          ++v;
          curc = nextc;
          nextc = cumt[v + 1];
        }
        symt[rr][sl] = (lo + v) | ((nextc - curc) << 8) | ((sl - curc) << 20);
      }
      continue;
    }
    const uint32_t slot0 = 64 * lane;
    uint32_t a = 0, z = tcount - 1;  // largest i with cumt[i] <= slot0
    while (a < z) {
      const uint32_t mid = (a + z + 1) / 2;
      if (cumt[mid] <= slot0) a = mid;
      else z = mid - 1;
    }
    uint32_t v = a, nextc = cumt[a + 1];
    uint32_t* lw = reinterpret_cast<uint32_t*>(&lut[rr][slot0]);
    for (uint32_t q4 = 0; q4 < 16; ++q4) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t sl = slot0 + 4 * q4 + b;
        while (nextc <= sl) {
          ++v;
          nextc = cumt[v + 1];
        }
        word |= (lo + v) << (8 * b);
      }
      lw[q4] = word;
    }
  }
  wave_sync();
  // ---- word rings: four slots of 256 words, half h of the stream's words in
  // slot h & 3, then a copy of slot 0's first 64 words; halves 0..2 resident
  // and half 3 loaded into registers
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    staged[rr] = make_uint2(0, 0);
    if (rr >= nr || nwords[rr] == 0) continue;
    const uint2 h0 = load_half(wp[rr], nwords[rr], 0);
    *reinterpret_cast<uint2*>(&ring[rr][4 * lane]) = h0;
    if (lane < kMirror / 4) *reinterpret_cast<uint2*>(&ring[rr][kDecRing + 4 * lane]) = h0;
    *reinterpret_cast<uint2*>(&ring[rr][kHalf + 4 * lane]) = load_half(wp[rr], nwords[rr], 1);
    *reinterpret_cast<uint2*>(&ring[rr][2 * kHalf + 4 * lane]) = load_half(wp[rr], nwords[rr], 2);
    staged[rr] = load_half(wp[rr], nwords[rr], 3);
  }
  wave_sync();

  // ---- main loop: 8 steps (512 symbols) per block
  const bool vec = t.vec16 != 0;
  uint8_t* dst = job.dst + c * t.chunk_bytes;
  const uint32_t steps = (n + 63) / 64;
  const uint32_t full = n / 64;  // steps in which every lane decodes a symbol
  const uint32_t nblk = (steps + 7) / 8;
  // RAW bytes for block b are loaded while block b-2 decodes.  Non-RAW
  // streams read 8 bytes of the directory (always inside the blob) and never
  // use them, so the loads carry no branch.
  // Deltas: a ZRUN stream was expanded by k_zrun_expand into its slot of
  // zbuf and is read like a RAW one.
  const uint8_t* rbase[E];
  uint32_t rlim[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const bool zr = DELTA && mode[k] == LTC_MODE_ZRUN;
    const bool raw = mode[k] == LTC_MODE_RAW || zr;
    rbase[k] = zr ? t.zbuf + (g * E + k) * (uint64_t)t.zstride : raw ? blob + off[k] : blob + kHeader;
    rlim[k] = raw ? n : 0u;
  }
  uint64_t rawv[E], rawm[E];
#pragma unroll
  for (int k = 0; k < E; ++k) {
    rawv[k] = load_raw8(rbase[k], 8 * lane, rlim[k]);
    rawm[k] = load_raw8(rbase[k], 512 + 8 * lane, rlim[k]);
  }

  // A block's decoded symbols go to its stream's dead ring slot (the slot the
  // next refill writes, which no ring read touches before then) in element
  // order, so output lane l finds the symbols of its elements 8l .. 8l+7 as
  // 8 consecutive bytes.
  auto stage_of = [&](int rr) __attribute__((always_inline)) -> uint8_t* {
    return reinterpret_cast<uint8_t*>(&ring[rr][kHalf * ((hcur[rr] + 3) & 3)]);
  };
  auto stage_bytes = [&](int rr) __attribute__((always_inline)) -> uint64_t {
    return *reinterpret_cast<const uint64_t*>(stage_of(rr) + 8 * lane);
  };
  // The ring word at position pos + (renormalising lanes below this one):
  // (pos mod 1024) + rank < 1024 + 64, and the copy of slot 0 after the ring
  // covers the positions that wrap.
  auto ring_word = [&](int rr, uint64_t mask) __attribute__((always_inline)) -> uint32_t {
    return *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(ring[rr]) +
                                              ((lanes_below(mask) + (pos[rr] & (kDecRing - 1))) << 1));
  };

  // One decoding step of coded stream rr.  Every lane reads a ring word and
  // keeps it only if it renormalises, so there is no branch; a read past W
  // cannot go unnoticed because it leaves pos > W for the end check.
  auto dstep = [&](auto guarded, int rr, int q) __attribute__((always_inline)) {
    constexpr bool G = decltype(guarded)::value;
    const bool active = !G || 64 * full + lane < n;
    const uint32_t xs = x[rr];
    const uint32_t sl = xs & (kTotal - 1);
    uint32_t v, xd;
    if constexpr (FUSED) {
      const uint32_t e = symt[rr][sl];
      v = e & 0xFFu;
      xd = __umul24((e >> 8) & 0xFFFu, xs >> 12) + (e >> 20);
    } else {
      v = lut[rr][sl];
      const uint32_t e = symt[rr][v];
      xd = __umul24(e & 0xFFFFu, xs >> 12) + sl - (e >> 16);
    }
    const bool need = active && xd < kRansLow;
    const uint64_t mask = ballot(need);
    uint32_t wv = ring_word(rr, mask);
    asm volatile("" : "+v"(wv));  // keep the read unconditional (no exec branch)
    const uint32_t xn = need ? (xd << 16) | wv : xd;
    x[rr] = active ? xn : xs;
    pos[rr] += (uint32_t)__popcll(mask);
    stage_of(rr)[64 * q + lane] = (uint8_t)v;
  };
  // the multi-table instantiations run only chunks with 2 or more coded
  // streams; with two table slots that is exactly 2
  const int nrun = MAXR == 2 ? 2 : nr;
  // Step q of every coded stream of a multi-stream chunk (full steps only),
  // phase by phase: the slot-table reads of all streams, then their symbol
  // reads, then their state updates and ring reads, so the streams' LDS
  // latencies overlap instead of adding up.  Same arithmetic as dstep.
  auto dstep_all = [&](int q) __attribute__((always_inline)) {
    static_assert(MAXR == 1 || MAXR == 2 || MAXR == 4, "table slots");
    uint32_t xs[MAXR], sl[MAXR], v[MAXR], e[MAXR], xd[MAXR], wv[MAXR];
    uint64_t mask[MAXR];
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr) wv[rr] = 0;
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr) {
      if (rr >= nrun) continue;
      xs[rr] = x[rr];
      sl[rr] = xs[rr] & (kTotal - 1);
      v[rr] = lut[rr][sl[rr]];
    }
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr)
      if (rr < nrun) e[rr] = symt[rr][v[rr]];
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr) {
      if (rr >= nrun) continue;
      xd[rr] = __umul24(e[rr] & 0xFFFFu, xs[rr] >> 12) + sl[rr] - (e[rr] >> 16);
      mask[rr] = ballot(xd[rr] < kRansLow);
      wv[rr] = ring_word(rr, mask[rr]);
    }
    // keep the reads unconditional (one barrier for all streams)
    if constexpr (MAXR == 2) asm volatile("" : "+v"(wv[0]), "+v"(wv[1]));
    if constexpr (MAXR == 4) asm volatile("" : "+v"(wv[0]), "+v"(wv[1]), "+v"(wv[2]), "+v"(wv[3]));
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr) {
      if (rr >= nrun) continue;
      x[rr] = xd[rr] < kRansLow ? (xd[rr] << 16) | wv[rr] : xd[rr];
      pos[rr] += (uint32_t)__popcll(mask[rr]);
      stage_of(rr)[64 * q + lane] = (uint8_t)v[rr];
    }
  };
  // Ring refill, once per block, after the block's symbols have been read
  // from the stage: halves hcur .. hcur+2 are resident and pos <
  // 256*(hcur+1) at every check, and a block reads at most 512 words, so no
  // read leaves the resident halves and at most two halves retire per check.
  // A retired half's successor (hcur+3, loaded a retirement ahead) goes to
  // the dead slot, and the next half is loaded into registers.
  auto refill = [&](int rr) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      if (pos[rr] >= kHalf * (hcur[rr] + 1)) {
        const uint32_t slot = (hcur[rr] + 3) & 3;
        wave_sync();
        *reinterpret_cast<uint2*>(&ring[rr][kHalf * slot + 4 * lane]) = staged[rr];
        if (slot == 0 && lane < kMirror / 4)
          *reinterpret_cast<uint2*>(&ring[rr][kDecRing + 4 * lane]) = staged[rr];
        staged[rr] = load_half(wp[rr], nwords[rr], hcur[rr] + 4);
        ++hcur[rr];
        wave_sync();
      }
    }
  };
  // Elements 8 lane .. 8 lane + 7 of the current block, from the stage, the
  // RAW bytes (rawv) and the constants, as 2E little-endian words.  PAT: the
  // top stream is the coded one and every other stream is RAW.
  auto assemble = [&](uint32_t* ow, auto patc) __attribute__((always_inline)) {
    constexpr bool PAT = decltype(patc)::value;
    uint32_t pl[2][E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
      uint64_t v;
      if (PAT) v = k == E - 1 ? stage_bytes(0) : rawv[k];
      else if (mode[k] == LTC_MODE_RANS) {
        if constexpr (MAXR == 1) {
          v = stage_bytes(0);
        } else {  // a static slot index keeps the per-stream registers out of memory
          v = 0;
#pragma unroll
          for (int rr = 0; rr < MAXR; ++rr)
            if (slot_of[k] == rr) v = stage_bytes(rr);
        }
      }
      else if (mode[k] == LTC_MODE_RAW || (DELTA && mode[k] == LTC_MODE_ZRUN)) v = rawv[k];
      else v = 0x0101010101010101ull * cval[k];
      pl[0][k] = (uint32_t)v;
      pl[1][k] = (uint32_t)(v >> 32);
    }
    planes_to_words<DT>(pl[0], ow);
    planes_to_words<DT>(pl[1], ow + E);
  };
  // vector store of elements 8 lane .. 8 lane + 7 of block b (streaming:
  // nothing reads them back)
  auto store_full = [&](uint32_t b, const uint32_t* ow) __attribute__((always_inline)) {
    uint8_t* op = dst + (uint64_t)(512 * b + 8 * lane) * E;
    if constexpr (E == 1) {
      store_nt8(op, ow[0], ow[1]);
    } else if constexpr (E == 2) {
      store_nt16(op, ow[0], ow[1], ow[2], ow[3]);
    } else {
      store_nt16(op, ow[0], ow[1], ow[2], ow[3]);
      store_nt16(op + 16, ow[4], ow[5], ow[6], ow[7]);
    }
  };
  uint32_t obuf[4][2 * E];

  // Fast loop: the full blocks of an aligned chunk with one coded stream.
  // One counter covers loads and stores on this ISA and a wait on a load
  // waits for every older access too, so each iteration issues the same
  // memory operations in the same order -- the refill load (only when a ring
  // half retires), the RAW loads for block b+2, then the store of block b-1
  // -- and the compiler's wait at the next refill or RAW use leaves that
  // younger store in flight.  (Refill checks every 4 steps, with output
  // stores in bursts, made those waits drain the stores: 0.75 against 0.64
  // ms for 28 BF16 tensors.)
  const uint32_t nfb = (MAXR == 1 && vec && nr == 1) ? full / 8 : 0u;
  auto fblock = [&](uint32_t b, auto subc, auto prevc, auto patc) __attribute__((always_inline)) {
    constexpr int SUB = decltype(subc)::value;
    constexpr bool PREV = decltype(prevc)::value;
    constexpr bool PAT = decltype(patc)::value;
    const uint32_t e0 = 512 * b + 8 * lane;
    uint2 bv[E];
    if constexpr (DELTA) {  // the base bytes of this block's elements
      const uint8_t* bp = job.base + c * t.chunk_bytes + (uint64_t)e0 * E;
#pragma unroll
      for (int q = 0; q < E; ++q) bv[q] = *reinterpret_cast<const uint2*>(bp + 8 * q);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) dstep(std::false_type{}, 0, q);
    wave_sync();
    uint32_t* ow = obuf[SUB];
    assemble(ow, patc);
    if constexpr (DELTA) {  // the decoded bytes are the delta: XOR the base back in
#pragma unroll
      for (int q = 0; q < E; ++q) {
        ow[2 * q] ^= bv[q].x;
        ow[2 * q + 1] ^= bv[q].y;
      }
    }
    refill(0);
    uint64_t rawn[E];
#pragma unroll
    for (int k = 0; k < E; ++k)
      rawn[k] = (PAT && k == E - 1) ? 0ull : load_raw8(rbase[k], e0 + 1024, rlim[k]);
    if constexpr (PREV) store_full(b - 1, obuf[SUB ^ 1]);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      rawv[k] = rawm[k];
      rawm[k] = rawn[k];
    }
    wave_sync();
  };
  auto fast_loop = [&](auto patc) __attribute__((always_inline)) {
    fblock(0, std::integral_constant<int, 0>{}, std::false_type{}, patc);
    uint32_t b = 1;
    for (; b + 1 < nfb; b += 2) {
      fblock(b, std::integral_constant<int, 1>{}, std::true_type{}, patc);
      fblock(b + 1, std::integral_constant<int, 0>{}, std::true_type{}, patc);
    }
    if (b < nfb) fblock(b, std::integral_constant<int, 1>{}, std::true_type{}, patc);
    if ((nfb - 1) & 1) store_full(nfb - 1, obuf[1]);
    else store_full(nfb - 1, obuf[0]);
  };
  if (nfb > 0) {
    // the pattern of BF16 and FP16 weights (coded exponent byte, RAW rest)
    // gets a copy of the loop without per-stream mode selection
    if constexpr (E == 2) {
      if (mode[0] == LTC_MODE_RAW && mode[1] == LTC_MODE_RANS) fast_loop(std::true_type{});
      else fast_loop(std::false_type{});
    } else {
      fast_loop(std::false_type{});
    }
  }

  // General loop: the remaining blocks (all of them for chunks with several
  // coded streams, none or only RAW/CONST streams, unaligned output, and the
  // partial block of a ragged chunk).  Output of NB blocks is stored together,
  // so the waits for loads drain store bursts less often.
  constexpr int NB = 4;
  auto block = [&](uint32_t b, auto subc) __attribute__((always_inline)) {
    constexpr int SUB = decltype(subc)::value;
    const uint32_t e0 = 512 * b + 8 * lane;
    uint64_t rawn[E];
#pragma unroll
    for (int k = 0; k < E; ++k) rawn[k] = load_raw8(rbase[k], e0 + 1024, rlim[k]);
    if (MAXR > 1 && 8 * (b + 1) <= full) {  // several streams, every step full
#pragma unroll
      for (int q = 0; q < 8; ++q) dstep_all(q);
    } else {
#pragma unroll
      for (int rr = 0; rr < MAXR; ++rr) {
        if (rr >= nr) continue;
        if (8 * (b + 1) <= full) {  // every step of the block is full
#pragma unroll
          for (int q = 0; q < 8; ++q) dstep(std::false_type{}, rr, q);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t step = 8 * b + q;
            if (step >= steps) continue;  // past the end: its byte is never written out
            if (step < full) dstep(std::false_type{}, rr, q);
            else dstep(std::true_type{}, rr, q);
          }
        }
      }
    }
    wave_sync();
    if (e0 < n) {
      uint32_t* ow = obuf[SUB];
      assemble(ow, std::false_type{});
      if constexpr (DELTA) {  // the decoded bytes are the delta: XOR the base back in
        const uint8_t* bp = job.base + c * t.chunk_bytes + (uint64_t)e0 * E;
        if (vec && e0 + 8 <= n) {
#pragma unroll
          for (int q = 0; q < 2 * E; q += 2) {
            const uint2 bv = *reinterpret_cast<const uint2*>(bp + 4 * q);
            ow[q] ^= bv.x;
            ow[q + 1] ^= bv.y;
          }
        } else {  // unrolled over the largest count, so ow stays in registers
          const uint32_t nb = (n - e0 < 8 ? n - e0 : 8) * E;
#pragma unroll
          for (uint32_t i = 0; i < 8 * E; ++i)
            if (i < nb) ow[i / 4] ^= (uint32_t)bp[i] << (8 * (i & 3));
        }
      }
      if (!(vec && e0 + 8 <= n)) {  // a ragged or unaligned block: bytes, now
        uint8_t* op = dst + (uint64_t)e0 * E;
        const uint32_t nb = (n - e0 < 8 ? n - e0 : 8) * E;
#pragma unroll
        for (uint32_t i = 0; i < 8 * E; ++i)
          if (i < nb) op[i] = (uint8_t)(ow[i / 4] >> (8 * (i & 3)));
      }
    }
    // the stage has been read: the dead slots may take the refills
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr)
      if (rr < nr) refill(rr);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      rawv[k] = rawm[k];
      rawm[k] = rawn[k];
    }
    wave_sync();
  };
  auto store_block = [&](uint32_t b, auto subc) __attribute__((always_inline)) {
    constexpr int SUB = decltype(subc)::value;
    const uint32_t e0 = 512 * b + 8 * lane;
    if (e0 < n && vec && e0 + 8 <= n) store_full(b, obuf[SUB]);
  };
  for (uint32_t b = nfb; b < nblk; b += NB) {
    static_for<NB>([&](auto i) {
      if (b + i < nblk) block(b + i, i);
    });
    static_for<NB>([&](auto i) {
      if (b + i < nblk) store_block(b + i, i);
    });
  }
  // ---- end checks: every coded stream consumed exactly its words and
  // returned to the initial state
  bool endbad = false;
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    if (rr >= nr) continue;
    endbad |= pos[rr] != nwords[rr] || x[rr] != kRansLow;
  }
  if (ballot(endbad) != 0 && lane == 0) *job.status = LTC_ERR_CORRUPT;
}

// Deltas: one workgroup per stream of the launch's chunks; a ZRUN payload is
// checked field by field and expanded into the stream's zbuf slot (the
// decoder then reads it like a RAW stream).  Any inconsistency is CORRUPT.
template <int DT>
__global__ __launch_bounds__(256) void k_zrun_expand(DTable t) {
  constexpr int E = Dt<DT>::E;
  __shared__ uint32_t red[8];
  const uint64_t s = t.c_begin * E + blockIdx.x;
  const uint64_t g = s / E;
  const int k = (int)(s % E);
  const int j = find_job(t, g);
  const DJob& job = t.jobs[j];
  const uint64_t c = g - job.chunk0;
  const uint32_t n = c + 1 == job.nchunks ? job.n_tail : t.n_full;
  const uint4 e = reinterpret_cast<const uint4*>(job.blob + kHeader)[c * E + k];
  if ((e.w & 0xFFu) != LTC_MODE_ZRUN) return;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid / 64;
  const uint64_t B = job.blob_nbytes;
  const uint64_t off = (uint64_t)e.x | ((uint64_t)e.y << 32);
  const uint32_t size = e.z;
  const uint32_t nb = (n + 63) / 64;
  bool bad = size < 16 || off > B || size > B - off || (off & 15);
  const uint8_t* pl = job.blob + off;
  uint32_t nnz = 0, nblk = 0, l2 = 0, lit = 0;
  if (!bad) {
    const uint4 h = *reinterpret_cast<const uint4*>(pl);
    nnz = h.x;
    nblk = h.y;
    l2 = 16u + (uint32_t)align16((nb + 7) / 8);
    lit = l2 + (uint32_t)align16(8ull * min(nblk, nb));
    bad = h.z != 0 || h.w != 0 || nblk > nb || nnz > n || (uint64_t)lit + nnz != size;
  }
  if (!bad) {  // pads: bitmap bits past the last block, bitmap pad, mask pad
    bool pb = false;
    for (uint32_t i = 16 + nb / 8 + tid; i < l2; i += 256) {
      const uint32_t v = pl[i];
      pb |= (i == 16 + nb / 8 && (nb & 7)) ? (v >> (nb & 7)) != 0 : v != 0;
    }
    for (uint32_t i = l2 + 8 * nblk + tid; i < lit; i += 256) pb |= pl[i] != 0;
    bad = __syncthreads_or(pb) != 0;
  }
  if (bad) {
    if (tid == 0) *job.status = LTC_ERR_CORRUPT;
    return;
  }
  uint8_t* out = t.zbuf + s * (uint64_t)t.zstride;
  const uint8_t* l2p = pl + l2;
  const uint8_t* lp = pl + lit;
  uint32_t run_blk = 0, run_lit = 0;
  bool err = false;
  for (uint32_t r0 = 0; r0 < nb; r0 += 256) {
    const uint32_t b = r0 + tid;
    const bool set = b < nb && ((pl[16 + b / 8] >> (b & 7)) & 1u);
    const uint64_t bal = ballot(set);
    if (lane == 63) red[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t blk_before = run_blk, blk_round = 0;
    for (uint32_t q = 0; q < 4; ++q) {
      if (q < wave) blk_before += red[q];
      blk_round += red[q];
    }
    const uint32_t rank = lanes_below_plus(bal, blk_before);
    uint64_t mask = 0;
    if (set) {
      if (rank < nblk) mask = *reinterpret_cast<const uint64_t*>(l2p + 8 * rank);
      err |= mask == 0 || (64 * b + 64 > n && (mask >> (n - 64 * b)) != 0);
    }
    const uint32_t pc = (uint32_t)__popcll(mask);
    const uint32_t lit_below = wave_exclusive_scan_u32(pc);
    __syncthreads();
    if (lane == 63) red[4 + wave] = lit_below + pc;
    __syncthreads();
    uint32_t lit_before = run_lit, lit_round = 0;
    for (uint32_t q = 0; q < 4; ++q) {
      if (q < wave) lit_before += red[4 + q];
      lit_round += red[4 + q];
    }
    if (b < nb) {
      uint32_t o = lit_before + lit_below;
      for (uint32_t i = 0; i < 64 && 64 * b + i < n; ++i) {
        uint8_t v = 0;
        if ((mask >> i) & 1u) {
          if (o < nnz) v = lp[o];
          ++o;
          err |= v == 0;
        }
        out[64 * b + i] = v;
      }
    }
    run_blk += blk_round;
    run_lit += lit_round;
    __syncthreads();
  }
  err |= run_blk != nblk || run_lit != nnz;
  if (__syncthreads_or(err) && tid == 0) *job.status = LTC_ERR_CORRUPT;
}

__global__ void k_status_init(DTable t) {
  const uint32_t j = threadIdx.x;
  if (j < t.count) *t.jobs[j].status = LTC_OK;
}

template <int DT, bool DELTA>
static hipError_t launch_decompress_d(DTable t, hipStream_t st, const hipEvent_t* ev, uint64_t c_begin,
                                      uint64_t c_end, bool init_status) {
  constexpr int E = Dt<DT>::E;
  t.c_begin = c_begin;
  t.c_end = c_end;
  const uint64_t n = c_end - c_begin;
  const dim3 dgrid((uint32_t)((n + kDecWaves - 1) / kDecWaves)), dblock(64 * kDecWaves);
  if (init_status) hipLaunchKernelGGL(k_status_init, dim3(1), dim3(64), 0, st, t);
  if (DELTA && n) hipLaunchKernelGGL(k_zrun_expand<DT>, dim3((uint32_t)(n * E)), dim3(256), 0, st, t);
  record(ev, 0, st);
  if (n && n <= kDecFusedMaxChunks) hipLaunchKernelGGL((k_decode<DT, 1, DELTA, true>), dgrid, dblock, 0, st, t);
  else if (n) hipLaunchKernelGGL((k_decode<DT, 1, DELTA>), dgrid, dblock, 0, st, t);
  record(ev, 1, st);
  if constexpr (E > 1) {
    if (n) hipLaunchKernelGGL((k_decode<DT, E, DELTA>), dgrid, dblock, 0, st, t);
  }
  record(ev, 2, st);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_decompress_t(DTable t, hipStream_t st, const hipEvent_t* ev, uint64_t c_begin,
                                      uint64_t c_end, bool init_status) {
  return t.delta ? launch_decompress_d<DT, true>(t, st, ev, c_begin, c_end, init_status)
                 : launch_decompress_d<DT, false>(t, st, ev, c_begin, c_end, init_status);
}

hipError_t launch_decompress_range(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev,
                                   uint64_t c_begin, uint64_t c_end, bool init_status) {
  switch (dtype) {
    case LTC_U8: return launch_decompress_t<LTC_U8>(t, st, ev, c_begin, c_end, init_status);
    case LTC_BF16: return launch_decompress_t<LTC_BF16>(t, st, ev, c_begin, c_end, init_status);
    case LTC_FP16: return launch_decompress_t<LTC_FP16>(t, st, ev, c_begin, c_end, init_status);
    case LTC_FP32: return launch_decompress_t<LTC_FP32>(t, st, ev, c_begin, c_end, init_status);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decompress(int dtype, const DTable& t, hipStream_t st, const hipEvent_t* ev) {
  return launch_decompress_range(dtype, t, st, ev, 0, t.total_chunks, true);
}

}  // namespace ltc
