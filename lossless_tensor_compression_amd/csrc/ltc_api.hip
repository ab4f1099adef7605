// ltc_api.hip -- host side of the C ABI declared in include/ltc.h:
// argument checks, sizes, workspace carving, header parsing and launches.
// Nothing here allocates device memory or synchronises.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "ltc_host.h"
#include "ltc_internal.h"
#include "ltc_launch.h"

// Workspace of ltc_compress_noalloc: one copy on each GPU the library runs
// on, held until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in for the device symbol); it uses
// the per-device pointer from hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) uint8_t scratch[LTC_NOALLOC_SCRATCH_BYTES];

namespace ltc {
namespace {

constexpr uint64_t kAlign = 256;
constexpr uint32_t kWordsGranule = 1024;

// ---- pipelined compression
// A compress call over at least kPipeMinChunks chunks splits them into
// kPipeGroups chunk-ordered groups.  Group 0 runs on the caller's stream, the
// others on internal streams forked from it and joined back to it, so one
// group's compute-bound encoding overlaps another's memory-bound histogram and
// packing.  The groups' scans run in chunk order (each waits for the previous
// one), so offsets and blobs are the same as with one group.  The streams
// (default priority, non-blocking) and events are created once per device on
// first use and kept until the process ends; the enqueue is serialised.
// Measured on 28 BF16 tensors (13,312 chunks): 2 groups 1.50 ms, 4 groups
// 1.56 ms, one stream 1.60 ms; with the checksums computed in k_pack, 2
// groups 1.60 ms against 1.66 on one stream.  Below 4096 chunks the fork,
// the cross-stream waits and the doubled launches cost more than the
// overlap: a 64 MiB FP32 tensor (512 chunks) compresses in 0.15 ms on one
// stream against 0.21 ms in two groups.  Top-last calls (no deltas) of that
// size do not pipeline: their encoder places the top streams' payloads
// itself (k_encode), whose look-back runs within one launch; on C3 that is
// 2-3% faster than the two groups (1.31 against 1.33-1.36 ms on one box, C5
// 5.49-5.52 against 5.65-5.68 ms).
constexpr int kPipeGroups = 2;
constexpr uint64_t kPipeMinChunks = 4096;

// ---- decoding blobs held in host memory
// The blobs are copied into device staging buffers in chunk-ordered groups
// on an internal stream (the DMA engines), and each group is decoded on the
// caller's stream as soon as its bytes have arrived, so decoding overlaps the
// transfer of the following groups.
// Every copy costs a fixed setup on the DMA engine, so groups are few and
// large: at most 8, of at least 16 MiB (C3's 1.15 GB of blobs load at 55 GB/s
// over the host link this way, against 50 GB/s with 64 groups of 4 MiB).
constexpr int kCopyGroupsMax = 8;
constexpr uint64_t kCopyGroupBytes = 16ull << 20;

struct PipeRes {
  hipStream_t s[kPipeGroups] = {};
  hipEvent_t fork = nullptr, scan[kPipeGroups] = {}, top[kPipeGroups] = {}, done[kPipeGroups] = {};
  hipEvent_t copied[kCopyGroupsMax] = {};
  bool ok = false;
};
std::mutex g_pipe_mu;
std::vector<PipeRes*> g_pipe;  // per device

// the current device's streams and events; call with g_pipe_mu held
PipeRes* pipe_res(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  hipDevice_t sdev = 0;  // the caller's stream must belong to the current device
  if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
  if ((int)g_pipe.size() <= dev) g_pipe.resize(dev + 1, nullptr);
  if (!g_pipe[dev]) {
    PipeRes* r = new PipeRes();
    bool ok = hipEventCreateWithFlags(&r->fork, hipEventDisableTiming) == hipSuccess;
    for (int g = 0; g < kPipeGroups; ++g) {
      if (g > 0) ok = ok && hipStreamCreateWithFlags(&r->s[g], hipStreamNonBlocking) == hipSuccess;
      ok = ok && hipEventCreateWithFlags(&r->scan[g], hipEventDisableTiming) == hipSuccess;
      ok = ok && hipEventCreateWithFlags(&r->top[g], hipEventDisableTiming) == hipSuccess;
      ok = ok && hipEventCreateWithFlags(&r->done[g], hipEventDisableTiming) == hipSuccess;
    }
    for (int g = 0; g < kCopyGroupsMax; ++g)
      ok = ok && hipEventCreateWithFlags(&r->copied[g], hipEventDisableTiming) == hipSuccess;
    r->ok = ok;
    g_pipe[dev] = r;
  }
  return g_pipe[dev]->ok ? g_pipe[dev] : nullptr;
}

// all chunks on one stream (one_stream, events, or a small call), or groups
// as above
hipError_t run_compress(CTable t, const CWork& w, hipStream_t stream, const hipEvent_t* ev,
                        bool one_stream) {
  const uint64_t total = t.total_chunks;
  t.c_begin = 0;
  t.c_end = total;
  // v2: every plane's table needs the histograms of all chunks, so they come
  // first, on the caller's stream, before the chunks are coded
  const bool staged = t.v2 != 0;
  if (staged) {
    const hipError_t err = launch_v2_tables(t, w, stream, ev);
    if (err != hipSuccess) return err;
  }
  // one stream: the two halves of the top-last schedule back to back
  auto whole = [&](const hipEvent_t* e) -> hipError_t {
    if (!t.top_last) return launch_compress(t, w, stream, e, nullptr, nullptr, staged);
    const hipError_t err = launch_compress_front(t, w, stream, e, nullptr, nullptr, staged);
    return err == hipSuccess ? launch_compress_back(t, w, stream, e, nullptr, nullptr) : err;
  };
  if (ev || one_stream || total < kPipeMinChunks || t.place) return whole(ev);
  std::lock_guard<std::mutex> lock(g_pipe_mu);
  PipeRes* r = pipe_res(stream);
  if (!r) return whole(nullptr);
  hipError_t err = hipEventRecord(r->fork, stream);
  for (int g = 1; g < kPipeGroups && err == hipSuccess; ++g) err = hipStreamWaitEvent(r->s[g], r->fork, 0);
  auto group = [&](int g) {
    CTable tg = t;
    tg.c_begin = total * g / kPipeGroups;
    tg.c_end = total * (g + 1) / kPipeGroups;
    return tg;
  };
  auto gstream = [&](int g) { return g == 0 ? stream : r->s[g]; };
  if (!t.top_last) {
    for (int g = 0; g < kPipeGroups && err == hipSuccess; ++g) {
      err = launch_compress(group(g), w, gstream(g), nullptr, g > 0 ? r->scan[g - 1] : nullptr, r->scan[g], staged);
      if (err == hipSuccess && g > 0) err = hipEventRecord(r->done[g], gstream(g));
    }
  } else {
    // front halves (lower scans chained in chunk order), then back halves:
    // the first top scan waits for the last lower scan, each later one for
    // the top scan before it.  Every event is recorded (enqueued) before a
    // wait on it is enqueued.
    for (int g = 0; g < kPipeGroups && err == hipSuccess; ++g)
      err = launch_compress_front(group(g), w, gstream(g), nullptr, g > 0 ? r->scan[g - 1] : nullptr,
                                  r->scan[g], staged);
    for (int g = 0; g < kPipeGroups && err == hipSuccess; ++g) {
      err = launch_compress_back(group(g), w, gstream(g), nullptr,
                                 g == 0 ? r->scan[kPipeGroups - 1] : r->top[g - 1], r->top[g]);
      if (err == hipSuccess && g > 0) err = hipEventRecord(r->done[g], gstream(g));
    }
  }
  for (int g = 1; g < kPipeGroups && err == hipSuccess; ++g) err = hipStreamWaitEvent(stream, r->done[g], 0);
  return err;
}

// ---- the scratch array of ltc_compress_noalloc
// Its device address, looked up once per device (with that device current)
// on the first call there, and kept; a fixed table, so no call allocates.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// the current device's scratch address, or null (stream of another device,
// or the lookup failed: *err tells which)
void* scratch_ptr(hipStream_t stream, int* err) {
  int dev = 0;
  *err = LTC_ERR_HIP;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  *err = LTC_ERR_INVALID_ARGUMENT;
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  hipDevice_t sdev = 0;
  if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = LTC_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

uint32_t gf2_mulmod_host(uint32_t a, uint32_t b) {
  uint32_t r = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) r ^= b;
    b = (b >> 1) ^ (0xEDB88320u & (0u - (b & 1u)));
  }
  return r;
}

// v * x^-1 mod P (undoes one step of v * x = (v >> 1) ^ (P if v & 1): the
// reflected polynomial has its top bit set, so that bit of the product is
// the bit v lost)
uint32_t div_x(uint32_t d) {
  const uint32_t low = d >> 31;
  return ((d ^ (0xEDB88320u & (0u - low))) << 1) | low;
}

// x^(-8*16*j) mod P for j = 0..63
const uint32_t* xinv_table() {
  static const std::vector<uint32_t> tab = [] {
    std::vector<uint32_t> v(64);
    uint32_t r = 0x80000000u;  // 1
    for (int j = 0; j < 64; ++j) {
      v[j] = r;
      for (int k = 0; k < 128; ++k) r = div_x(r);
    }
    return v;
  }();
  return tab.data();
}

// x^(8n) mod P in the reflected representation (bit 31 - d = x^d)
uint32_t xpow8(uint64_t n) {
  uint32_t r = 0x80000000u, sq = 0x00800000u;
  while (n) {
    if (n & 1) r = gf2_mulmod_host(r, sq);
    sq = gf2_mulmod_host(sq, sq);
    n >>= 1;
  }
  return r;
}


// Largest integer P with (double)P < theta * (double)n: cuZipNN 0.1.0, "API":
// coding is kept only when the coded size is under that fraction of the raw one.
uint32_t p_max(uint64_t n, double theta) {
  const double lim = theta * (double)n;
  if (!(lim > 0.0)) return 0;
  double p = floor(lim);
  if (p >= lim) p -= 1.0;
  return p < 0.0 ? 0u : (uint32_t)p;
}

int check_shape(uint64_t nbytes, int dtype, uint32_t chunk_bytes) {
  const uint32_t e = elem_bytes(dtype);
  if (!e) return LTC_ERR_UNSUPPORTED_DTYPE;
  if (nbytes % e) return LTC_ERR_INVALID_ARGUMENT;
  if (chunk_bytes < 8 || chunk_bytes > (1u << 24) || chunk_bytes % 8) return LTC_ERR_INVALID_ARGUMENT;
  const uint64_t k = nbytes / chunk_bytes + (nbytes % chunk_bytes != 0);  // no wrap for any N
  if (k >= (1ull << 32)) return LTC_ERR_INVALID_ARGUMENT;
  return LTC_OK;
}

// words per stream reserved in the workspace: enough for any threshold <= 1
uint32_t words_capacity(uint32_t chunk_bytes, uint32_t e) {
  const uint32_t n = chunk_bytes / e;
  const uint32_t pmax = n - 1;  // theta = 1
  const uint32_t w = pmax > kRansFixed ? (pmax - kRansFixed) / 2 + 1 : 1;
  return (uint32_t)round_up(w, kWordsGranule);
}

struct Layout {
  uint64_t sinfo, freq, hist, plane, ptab, pbase, zinfo, states, offsets, blobn, toprun, tstat, frames, words, total;
};

// frames: one u32 per KiB of every blob's bound (compress_with_crc32);
// hist, plane, ptab, pbase: format v2
Layout layout(uint64_t streams, int count, uint32_t wcap, uint64_t frames, uint32_t e) {
  Layout l;
  uint64_t cur = 0;
  l.sinfo = cur;   cur = round_up(cur + 16 * streams, kAlign);
  l.freq = cur;    cur = round_up(cur + 512 * streams, kAlign);
  l.hist = cur;    cur = round_up(cur + 1024 * streams, kAlign);
  l.plane = cur;   cur = round_up(cur + 2048ull * e * (uint64_t)count, kAlign);
  l.ptab = cur;    cur = round_up(cur + 512ull * e * (uint64_t)count, kAlign);
  l.pbase = cur;   cur = round_up(cur + 8 * (uint64_t)count, kAlign);
  l.zinfo = cur;   cur = round_up(cur + 8 * streams, kAlign);
  l.states = cur;  cur = round_up(cur + 256 * streams, kAlign);
  l.offsets = cur; cur = round_up(cur + 8 * streams, kAlign);
  l.blobn = cur;   cur = round_up(cur + 8 * (uint64_t)count, kAlign);
  l.toprun = cur;  cur = round_up(cur + 8 * (uint64_t)count, kAlign);
  l.tstat = cur;   cur = round_up(cur + 8 * streams, kAlign);  // one per chunk suffices
  l.frames = cur;  cur = round_up(cur + 4 * frames, kAlign);
  l.words = cur;   cur = round_up(cur + 2ull * wcap * streams, kAlign);
  l.total = cur;
  return l;
}

uint64_t bound_of(uint64_t nbytes, uint32_t e, uint32_t chunk_bytes) {
  const uint64_t k = (nbytes + chunk_bytes - 1) / chunk_bytes;
  if (k == 0) return kHeader;
  const uint64_t full = nbytes / chunk_bytes;
  const uint64_t tail = nbytes - full * chunk_bytes;
  uint64_t b = kHeader + kDirEntry * k * e + full * e * align16(chunk_bytes / e);
  if (tail) b += e * align16(tail / e);
  return b;
}

// v2 adds E table records of at most 16 + 2*256 bytes
uint64_t bound_flags(uint64_t nbytes, uint32_t e, uint32_t chunk_bytes, uint32_t flags) {
  return bound_of(nbytes, e, chunk_bytes) + ((flags & LTC_FLAG_SHARED_TABLES) ? 528ull * e : 0);
}

// frame slots for compress_with_crc32: enough for either format
uint64_t batch_frames(int count, const uint64_t* nbytes, uint32_t e, uint32_t chunk_bytes) {
  uint64_t f = 0;
  for (int i = 0; i < count; ++i)
    f += (bound_flags(nbytes[i], e, chunk_bytes, LTC_FLAG_SHARED_TABLES) + 1023) / 1024;
  return f;
}

int64_t batch_streams(int count, const uint64_t* nbytes, uint32_t e, uint32_t chunk_bytes) {
  uint64_t chunks = 0;
  for (int i = 0; i < count; ++i) chunks += (nbytes[i] + chunk_bytes - 1) / chunk_bytes;
  // grid limit: chunks * 256 work-items per launch must stay below 2^32
  if (chunks >= (1ull << 24)) return -1;
  return (int64_t)(chunks * e);
}

// checksums requested with a compress call (compress_with_crc32)
struct CrcReq {
  uint32_t chunk_bytes;      // K; 0: none
  uint32_t* const* outs;     // per tensor, ceil(bound / K) entries at least
  const uint64_t* caps;      // entries available per tensor
};

int compress_impl(int count, const void* const* srcs, const uint64_t* nbytes, int dtype,
                  uint32_t chunk_bytes, double theta, void* const* blobs, const uint64_t* caps,
                  uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes, hipStream_t stream,
                  const hipEvent_t* ev, const CrcReq& crc = CrcReq{0, nullptr, nullptr},
                  uint32_t flags = 0, const void* const* bases = nullptr) {
  if (count < 1 || count > kMaxJobs || !srcs || !nbytes || !blobs || !caps || !d_blob_nbytes)
    return LTC_ERR_INVALID_ARGUMENT;
  if (flags & ~(LTC_FLAG_SHARED_TABLES | LTC_FLAG_CALLER_STREAM_ONLY | LTC_FLAG_TOP_LAST |
                LTC_FLAG_PLACE_NO_WAIT))
    return LTC_ERR_INVALID_ARGUMENT;
  if (!(theta > 0.0 && theta <= 1.0)) return LTC_ERR_INVALID_ARGUMENT;
  const bool one_stream = (flags & LTC_FLAG_CALLER_STREAM_ONLY) != 0;
  const uint32_t e = elem_bytes(dtype);
  for (int i = 0; i < count; ++i) {
    const int rc = check_shape(nbytes[i], dtype, chunk_bytes);
    if (rc) return rc;
    if (!blobs[i] || (nbytes[i] && !srcs[i])) return LTC_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(srcs[i]) % e) return LTC_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(blobs[i]) % 16) return LTC_ERR_INVALID_ARGUMENT;
    if (caps[i] < bound_flags(nbytes[i], e, chunk_bytes, flags)) return LTC_ERR_CAPACITY;
    if (bases && nbytes[i] && (!bases[i] || reinterpret_cast<uintptr_t>(bases[i]) % e))
      return LTC_ERR_INVALID_ARGUMENT;
  }
  if (crc.chunk_bytes) {
    if (!crc.outs || !crc.caps) return LTC_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < count; ++i) {
      if (!crc.outs[i] || reinterpret_cast<uintptr_t>(crc.outs[i]) % 4) return LTC_ERR_INVALID_ARGUMENT;
      const uint64_t need =
          (bound_flags(nbytes[i], e, chunk_bytes, flags) + crc.chunk_bytes - 1) / crc.chunk_bytes;
      if (crc.caps[i] < need) return LTC_ERR_CAPACITY;
    }
  }
  const int64_t streams = batch_streams(count, nbytes, e, chunk_bytes);
  if (streams < 0) return LTC_ERR_INVALID_ARGUMENT;
  const uint32_t wcap = words_capacity(chunk_bytes, e);
  const Layout l = layout((uint64_t)streams, count, wcap, batch_frames(count, nbytes, e, chunk_bytes), e);
  if (!d_ws || ws_nbytes < l.total || reinterpret_cast<uintptr_t>(d_ws) % kAlign)
    return LTC_ERR_WORKSPACE;

  CTable t;
  memset(&t, 0, sizeof(t));
  t.count = (uint32_t)count;
  t.chunk_bytes = chunk_bytes;
  t.n_full = chunk_bytes / e;
  t.wcap = wcap;
  t.dtype = (uint32_t)dtype;
  t.v2 = (flags & LTC_FLAG_SHARED_TABLES) ? 1u : 0u;
  t.delta = bases ? 1u : 0u;
  t.top_last = (flags & LTC_FLAG_TOP_LAST) ? 1u : 0u;
  bool vec = chunk_bytes % 16 == 0;
  uint64_t chunk0 = 0;
  for (int i = 0; i < count; ++i) {
    CJob& jb = t.jobs[i];
    jb.src = static_cast<const uint8_t*>(srcs[i]);
    jb.base = bases ? static_cast<const uint8_t*>(bases[i]) : nullptr;
    jb.blob = static_cast<uint8_t*>(blobs[i]);
    jb.blob_nbytes_out = d_blob_nbytes + i;
    jb.nbytes = nbytes[i];
    jb.chunk0 = chunk0;
    jb.nchunks = (uint32_t)((nbytes[i] + chunk_bytes - 1) / chunk_bytes);
    const uint64_t tail_bytes = nbytes[i] - (uint64_t)(jb.nchunks ? jb.nchunks - 1 : 0) * chunk_bytes;
    jb.n_tail = (uint32_t)(tail_bytes / e);
    jb.pmax_full = p_max(t.n_full, theta);
    jb.pmax_tail = p_max(jb.n_tail, theta);
    chunk0 += jb.nchunks;
    if (nbytes[i] && reinterpret_cast<uintptr_t>(srcs[i]) % 16) vec = false;
    if (bases && nbytes[i] && reinterpret_cast<uintptr_t>(bases[i]) % 16) vec = false;
  }
  t.total_chunks = chunk0;
  t.vec16 = vec ? 1u : 0u;
  // top-last calls large enough to pipeline: k_encode places the top
  // streams' payloads instead, on one stream (a smaller call waits longer in
  // the look-back than packing takes)
  t.place = t.top_last && !bases && chunk0 >= kPipeMinChunks ? 1u : 0u;
  // device-clock ticks (100 MHz) a placing wave waits for the sizes before
  // its chunk: about 1 ms plus the time to code one chunk's stream
  t.place_wait = (flags & LTC_FLAG_PLACE_NO_WAIT) ? 0 : 100000ull + 2ull * t.n_full;
  uint8_t* ws = static_cast<uint8_t*>(d_ws);
  CWork w;
  w.sinfo = reinterpret_cast<uint32_t*>(ws + l.sinfo);
  w.freq = reinterpret_cast<uint16_t*>(ws + l.freq);
  w.hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  w.plane = reinterpret_cast<uint64_t*>(ws + l.plane);
  w.ptab = reinterpret_cast<uint16_t*>(ws + l.ptab);
  w.pbase = reinterpret_cast<uint64_t*>(ws + l.pbase);
  w.zinfo = reinterpret_cast<uint2*>(ws + l.zinfo);
  w.states = reinterpret_cast<uint32_t*>(ws + l.states);
  w.offsets = reinterpret_cast<uint64_t*>(ws + l.offsets);
  w.blob_nbytes = reinterpret_cast<uint64_t*>(ws + l.blobn);
  w.top_run = reinterpret_cast<uint64_t*>(ws + l.toprun);
  w.tstat = reinterpret_cast<uint64_t*>(ws + l.tstat);
  w.words = reinterpret_cast<uint16_t*>(ws + l.words);
  if (!crc.chunk_bytes) return run_compress(t, w, stream, ev, one_stream) == hipSuccess ? LTC_OK : LTC_ERR_HIP;

  // compress_with_crc32: when checksum chunks are whole 1 KiB frames, k_scan
  // and k_pack accumulate the remainders of the blob's frames as they write
  // it and k_crc_frames chains them per chunk; otherwise k_crc32 reads the
  // finished blobs back.
  const uint64_t K = crc.chunk_bytes;
  // deltas write ZRUN payloads byte by byte: their blobs are read back.  So
  // are top-last blobs, whose RAW streams k_encode writes: checksumming them
  // in k_pack (C3: 0.44 against 0.18 ms) costs more than reading the blob
  // once more with k_crc32's conflict-free tables (0.24 ms).
  const bool fused = crc_frames_usable(K) && !bases && !(flags & LTC_FLAG_TOP_LAST);
  uint32_t* frames = reinterpret_cast<uint32_t*>(ws + l.frames);
  CrcArgs a;
  memset(&a, 0, sizeof(a));
  a.count = (uint32_t)count;
  a.chunk_bytes = K;
  a.seg = round_up(K, 256) / 64;
  for (int lv = 0; lv < 6; ++lv) a.lvl[lv] = xpow8(a.seg << lv);
  a.x1k = xpow8(1024);
  memcpy(a.xinv, xinv_table(), sizeof(a.xinv));
  if (fused) {
    t.crc = 1;
    t.crc_frames = (uint32_t)(K / 1024);
    t.crc_x1k = xpow8(1024);
    for (int k = 0; k < 64; ++k) t.crc_pos[k] = xpow8(16ull * (63 - k));
  }
  uint64_t fcur = 0, ccur = 0;
  for (int i = 0; i < count; ++i) {
    const uint64_t bound = bound_flags(nbytes[i], e, chunk_bytes, flags);
    t.jobs[i].frames = frames + fcur;
    CrcJob& jb = a.jobs[i];
    jb.src = t.jobs[i].blob;
    jb.out = crc.outs[i];
    jb.len = d_blob_nbytes + i;
    jb.frames = fused ? frames + fcur : nullptr;
    jb.chunk0 = ccur;
    jb.nchunks = (bound + K - 1) / K;
    fcur += (bound + 1023) / 1024;
    ccur += jb.nchunks;
  }
  a.total_chunks = ccur;
  hipError_t err = fused ? launch_zero_u32(frames, fcur, stream) : hipSuccess;
  if (err == hipSuccess) err = run_compress(t, w, stream, ev, one_stream);
  if (err == hipSuccess) err = fused ? launch_crc32_frames(a, stream) : launch_crc32(a, stream);
  if (ev) record(ev, 5, stream);
  return err == hipSuccess ? LTC_OK : LTC_ERR_HIP;
}

uint32_t rd_flags(const void* header) { return static_cast<const uint8_t*>(header)[27]; }

// Copies and decodes blobs held in host memory (t's blobs are the staging
// buffers; every header was checked).  Group g holds global chunks
// [T*g/G, T*(g+1)/G); its bytes of blob j are that tensor's directory (first
// group of the tensor) and the payloads from the first stream of its first
// chunk to the first stream of the next group's (or the blob's end), clamped
// to the blob; for a top-last blob, that span for its lower streams and
// another for its top streams (host_group_ranges).  The decoder validates every offset it uses, so a corrupt
// directory can only leave bytes of the staging buffer stale, never lead to
// an access outside it.
hipError_t decode_from_host(int dtype, const DTable& t, uint32_t e, const void* const* host_blobs,
                            hipStream_t stream) {
  const uint64_t T = t.total_chunks;
  if (T == 0) return launch_decompress_range(dtype, t, stream, nullptr, 0, 0, true);
  HostBlob hb[kMaxJobs];
  uint64_t total = 0;
  for (uint32_t j = 0; j < t.count; ++j) {
    const DJob& jb = t.jobs[j];
    hb[j] = HostBlob{static_cast<const uint8_t*>(host_blobs[j]), jb.blob_nbytes, jb.chunk0, jb.nchunks,
                     jb.top_last != 0};
    total += jb.blob_nbytes;
  }
  const uint64_t G = host_copy_groups(total, T, kCopyGroupBytes, kCopyGroupsMax);
  std::lock_guard<std::mutex> lock(g_pipe_mu);
  PipeRes* r = pipe_res(stream);
  if (!r) return hipErrorInvalidValue;
  hipStream_t cs = r->s[1];
  hipError_t err = hipEventRecord(r->fork, stream);
  if (err == hipSuccess) err = hipStreamWaitEvent(cs, r->fork, 0);
  HostRange rg[2 * kMaxJobs];
  for (uint64_t g = 0; g < G && err == hipSuccess; ++g) {
    const uint32_t nr = host_group_ranges(hb, t.count, e, T, G, g, rg);
    for (uint32_t q = 0; q < nr && err == hipSuccess; ++q) {
      const HostRange& x = rg[q];
      err = hipMemcpyAsync(const_cast<uint8_t*>(t.jobs[x.job].blob) + x.lo, hb[x.job].data + x.lo, x.hi - x.lo,
                           hipMemcpyHostToDevice, cs);
    }
    if (err == hipSuccess) err = hipEventRecord(r->copied[g], cs);
    if (err == hipSuccess) err = hipStreamWaitEvent(stream, r->copied[g], 0);
    if (err == hipSuccess)
      err = launch_decompress_range(dtype, t, stream, nullptr, T * g / G, T * (g + 1) / G, g == 0);
  }
  return err;
}

// host_blobs (optional): the whole blobs in host memory; blobs are then the
// device staging buffers they are copied into (stage_caps bytes each)
// bases (optional): the delta bases; every blob must then be a delta blob,
// and d_ws holds the expanded ZRUN streams (ltc_decompress_workspace_size)
int decompress_impl(int count, const void* const* headers, const void* const* blobs,
                    const uint64_t* blob_nbytes, void* const* dsts, const uint64_t* caps,
                    int32_t* d_status, hipStream_t stream, const hipEvent_t* ev,
                    const void* const* host_blobs = nullptr, const uint64_t* stage_caps = nullptr,
                    const void* const* bases = nullptr, void* d_ws = nullptr, uint64_t ws_nbytes = 0) {
  if (count < 1 || count > kMaxJobs || !headers || !blobs || !blob_nbytes || !dsts || !caps || !d_status)
    return LTC_ERR_INVALID_ARGUMENT;
  if (host_blobs && !stage_caps) return LTC_ERR_INVALID_ARGUMENT;
  DTable t;
  memset(&t, 0, sizeof(t));
  t.count = (uint32_t)count;
  int dtype = -1;
  uint32_t chunk_bytes = 0, e = 0;
  bool vec = true;
  uint64_t chunk0 = 0;
  for (int i = 0; i < count; ++i) {
    ltc_info info;
    const int rc = ltc_blob_info(headers[i], kHeader, &info);
    if (rc) return rc;
    if (i == 0) {
      dtype = info.dtype;
      chunk_bytes = info.chunk_bytes;
      e = info.elem_bytes;
    } else if (info.dtype != dtype || info.chunk_bytes != chunk_bytes) {
      return LTC_ERR_INVALID_ARGUMENT;
    }
    if (info.blob_nbytes != blob_nbytes[i]) return LTC_ERR_CORRUPT;
    if (caps[i] < info.nbytes) return LTC_ERR_CAPACITY;
    if (!blobs[i] || (info.nbytes && !dsts[i])) return LTC_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(blobs[i]) % 16) return LTC_ERR_INVALID_ARGUMENT;
    if (host_blobs && stage_caps[i] < info.blob_nbytes) return LTC_ERR_CAPACITY;
    // a delta blob needs its base, and a base needs a delta blob
    const bool delta = (rd_flags(headers[i]) & LTC_FLAG_DELTA) != 0;
    if (delta != (bases != nullptr)) return LTC_ERR_INVALID_ARGUMENT;
    if (delta && info.nbytes && (!bases[i] || reinterpret_cast<uintptr_t>(bases[i]) % e))
      return LTC_ERR_INVALID_ARGUMENT;
    DJob& jb = t.jobs[i];
    jb.base = delta ? static_cast<const uint8_t*>(bases[i]) : nullptr;
    if (delta && info.nbytes && reinterpret_cast<uintptr_t>(bases[i]) % 16) vec = false;
    jb.blob = static_cast<const uint8_t*>(blobs[i]);
    jb.dst = static_cast<uint8_t*>(dsts[i]);
    jb.status = d_status + i;
    jb.payload_base = info.payload_base;
    jb.v2 = info.version == 2 ? 1u : 0u;
    jb.top_last = (info.flags & LTC_FLAG_TOP_LAST) ? 1u : 0u;
    jb.blob_nbytes = info.blob_nbytes;
    jb.nbytes = info.nbytes;
    jb.chunk0 = chunk0;
    jb.nchunks = info.nchunks;
    const uint64_t tail_bytes = info.nbytes - (uint64_t)(info.nchunks ? info.nchunks - 1 : 0) * chunk_bytes;
    jb.n_tail = (uint32_t)(tail_bytes / e);
    chunk0 += info.nchunks;
    if (info.nbytes && reinterpret_cast<uintptr_t>(dsts[i]) % 16) vec = false;
  }
  if (chunk0 >= (1ull << 26)) return LTC_ERR_INVALID_ARGUMENT;  // 64 work-items per chunk
  t.chunk_bytes = chunk_bytes;
  t.n_full = chunk_bytes / e;
  t.vec16 = (vec && chunk_bytes % 16 == 0) ? 1u : 0u;
  t.total_chunks = chunk0;
  if (bases) {
    if (host_blobs) return LTC_ERR_INVALID_ARGUMENT;  // deltas are decoded from device blobs
    t.zstride = (uint32_t)align16(t.n_full);
    const uint64_t need = chunk0 * e * (uint64_t)t.zstride;
    if (need && (!d_ws || ws_nbytes < need)) return LTC_ERR_WORKSPACE;
    t.delta = 1;
    t.zbuf = static_cast<uint8_t*>(d_ws);
  }
  if (!host_blobs) return launch_decompress(dtype, t, stream, ev) == hipSuccess ? LTC_OK : LTC_ERR_HIP;
  return decode_from_host(dtype, t, e, host_blobs, stream) == hipSuccess ? LTC_OK : LTC_ERR_HIP;
}

}  // namespace
}  // namespace ltc

using namespace ltc;

extern "C" {

uint64_t ltc_compress_bound(uint64_t nbytes, int dtype, uint32_t chunk_bytes) {
  if (check_shape(nbytes, dtype, chunk_bytes)) return 0;
  return bound_of(nbytes, elem_bytes(dtype), chunk_bytes);
}

uint64_t ltc_compress_bound_ex(uint64_t nbytes, int dtype, uint32_t chunk_bytes, uint32_t flags) {
  if (check_shape(nbytes, dtype, chunk_bytes) ||
      (flags & ~(LTC_FLAG_SHARED_TABLES | LTC_FLAG_CALLER_STREAM_ONLY | LTC_FLAG_TOP_LAST |
                 LTC_FLAG_PLACE_NO_WAIT)))
    return 0;
  return bound_flags(nbytes, elem_bytes(dtype), chunk_bytes, flags);
}

int ltc_compress_batch_ex(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                          int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                          uint32_t flags, const void* const* h_base_ptrs, void* const* h_blob_ptrs,
                          const uint64_t* h_blob_capacity, uint64_t* d_blob_nbytes,
                          uint32_t checksum_chunk_bytes, uint32_t* const* h_crc_ptrs,
                          const uint64_t* h_crc_capacity, void* d_ws, uint64_t ws_nbytes,
                          hipStream_t stream, const hipEvent_t* h_events) {
  const CrcReq crc{checksum_chunk_bytes, h_crc_ptrs, h_crc_capacity};
  return compress_impl(count, h_src_ptrs, h_nbytes, dtype, chunk_bytes, passthrough_threshold,
                       h_blob_ptrs, h_blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, h_events,
                       crc, flags, h_base_ptrs);
}

int ltc_compress_delta(const void* d_src, const void* d_base, uint64_t nbytes, int dtype,
                       uint32_t chunk_bytes, double passthrough_threshold, uint32_t flags, void* d_blob,
                       uint64_t blob_capacity, uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                       hipStream_t stream) {
  if (!d_base) return LTC_ERR_INVALID_ARGUMENT;
  return ltc_compress_batch_ex(1, &d_src, &nbytes, dtype, chunk_bytes, passthrough_threshold, flags,
                               &d_base, &d_blob, &blob_capacity, d_blob_nbytes, 0, nullptr, nullptr,
                               d_ws, ws_nbytes, stream, nullptr);
}

int ltc_compress_workspace_size(uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                                uint64_t* ws_nbytes) {
  return ltc_compress_batch_workspace_size(1, &nbytes, dtype, chunk_bytes, ws_nbytes);
}

int ltc_compress_batch_workspace_size(int count, const uint64_t* h_nbytes, int dtype,
                                      uint32_t chunk_bytes, uint64_t* ws_nbytes) {
  if (count < 1 || count > kMaxJobs || !h_nbytes || !ws_nbytes) return LTC_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < count; ++i) {
    const int rc = check_shape(h_nbytes[i], dtype, chunk_bytes);
    if (rc) return rc;
  }
  const uint32_t e = elem_bytes(dtype);
  const int64_t streams = batch_streams(count, h_nbytes, e, chunk_bytes);
  if (streams < 0) return LTC_ERR_INVALID_ARGUMENT;
  *ws_nbytes = layout((uint64_t)streams, count, words_capacity(chunk_bytes, e),
                      batch_frames(count, h_nbytes, e, chunk_bytes), e).total;
  return LTC_OK;
}

int ltc_compress(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                 double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                 uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes, hipStream_t stream) {
  return compress_impl(1, &d_src, &nbytes, dtype, chunk_bytes, passthrough_threshold, &d_blob,
                       &blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, nullptr);
}

int ltc_compress_noalloc(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                         double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                         uint64_t* d_blob_nbytes, hipStream_t stream) {
  uint64_t need = 0;
  const int rc = ltc_compress_workspace_size(nbytes, dtype, chunk_bytes, &need);
  if (rc) return rc;
  if (need > LTC_NOALLOC_SCRATCH_BYTES) return LTC_ERR_WORKSPACE;
  int err = LTC_OK;
  void* ws = scratch_ptr(stream, &err);
  if (!ws) return err;
  return compress_impl(1, &d_src, &nbytes, dtype, chunk_bytes, passthrough_threshold, &d_blob,
                       &blob_capacity, d_blob_nbytes, ws, LTC_NOALLOC_SCRATCH_BYTES, stream, nullptr,
                       CrcReq{0, nullptr, nullptr}, LTC_FLAG_CALLER_STREAM_ONLY);
}

int ltc_compress_batch(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                       int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                       void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                       uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                       hipStream_t stream) {
  return compress_impl(count, h_src_ptrs, h_nbytes, dtype, chunk_bytes, passthrough_threshold,
                       h_blob_ptrs, h_blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, nullptr);
}

int ltc_compress_batch_prof(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                            int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                            void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                            uint64_t* d_blob_nbytes, void* d_ws, uint64_t ws_nbytes,
                            hipStream_t stream, const hipEvent_t* h_events) {
  return compress_impl(count, h_src_ptrs, h_nbytes, dtype, chunk_bytes, passthrough_threshold,
                       h_blob_ptrs, h_blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, h_events);
}

int ltc_compress_with_crc32(const void* d_src, uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                            double passthrough_threshold, void* d_blob, uint64_t blob_capacity,
                            uint64_t* d_blob_nbytes, uint32_t checksum_chunk_bytes, uint32_t* d_crc,
                            uint64_t crc_capacity, void* d_ws, uint64_t ws_nbytes,
                            hipStream_t stream) {
  if (checksum_chunk_bytes == 0) return LTC_ERR_INVALID_ARGUMENT;
  const CrcReq crc{checksum_chunk_bytes, &d_crc, &crc_capacity};
  return compress_impl(1, &d_src, &nbytes, dtype, chunk_bytes, passthrough_threshold, &d_blob,
                       &blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, nullptr, crc);
}

int ltc_compress_batch_with_crc32(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                                  int dtype, uint32_t chunk_bytes, double passthrough_threshold,
                                  void* const* h_blob_ptrs, const uint64_t* h_blob_capacity,
                                  uint64_t* d_blob_nbytes, uint32_t checksum_chunk_bytes,
                                  uint32_t* const* h_crc_ptrs, const uint64_t* h_crc_capacity,
                                  void* d_ws, uint64_t ws_nbytes, hipStream_t stream) {
  if (checksum_chunk_bytes == 0) return LTC_ERR_INVALID_ARGUMENT;
  const CrcReq crc{checksum_chunk_bytes, h_crc_ptrs, h_crc_capacity};
  return compress_impl(count, h_src_ptrs, h_nbytes, dtype, chunk_bytes, passthrough_threshold,
                       h_blob_ptrs, h_blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, nullptr, crc);
}

int ltc_compress_batch_with_crc32_prof(int count, const void* const* h_src_ptrs,
                                       const uint64_t* h_nbytes, int dtype, uint32_t chunk_bytes,
                                       double passthrough_threshold, void* const* h_blob_ptrs,
                                       const uint64_t* h_blob_capacity, uint64_t* d_blob_nbytes,
                                       uint32_t checksum_chunk_bytes, uint32_t* const* h_crc_ptrs,
                                       const uint64_t* h_crc_capacity, void* d_ws,
                                       uint64_t ws_nbytes, hipStream_t stream,
                                       const hipEvent_t* h_events) {
  if (checksum_chunk_bytes == 0 || !h_events) return LTC_ERR_INVALID_ARGUMENT;
  const CrcReq crc{checksum_chunk_bytes, h_crc_ptrs, h_crc_capacity};
  return compress_impl(count, h_src_ptrs, h_nbytes, dtype, chunk_bytes, passthrough_threshold,
                       h_blob_ptrs, h_blob_capacity, d_blob_nbytes, d_ws, ws_nbytes, stream, h_events,
                       crc);
}

int ltc_decompress(const void* h_header, const void* d_blob, uint64_t blob_nbytes, void* d_dst,
                   uint64_t dst_capacity, int32_t* d_status, hipStream_t stream) {
  return decompress_impl(1, &h_header, &d_blob, &blob_nbytes, &d_dst, &dst_capacity, d_status,
                         stream, nullptr);
}

int ltc_decompress_batch(int count, const void* const* h_headers, const void* const* h_blob_ptrs,
                         const uint64_t* h_blob_nbytes, void* const* h_dst_ptrs,
                         const uint64_t* h_dst_capacity, int32_t* d_status, hipStream_t stream) {
  return decompress_impl(count, h_headers, h_blob_ptrs, h_blob_nbytes, h_dst_ptrs, h_dst_capacity,
                         d_status, stream, nullptr);
}

int ltc_decompress_delta_workspace_size(int count, const void* const* h_headers, uint64_t* ws_nbytes) {
  if (count < 1 || count > kMaxJobs || !h_headers || !ws_nbytes) return LTC_ERR_INVALID_ARGUMENT;
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) {
    ltc_info info;
    const int rc = ltc_blob_info(h_headers[i], kHeader, &info);
    if (rc) return rc;
    total += (uint64_t)info.nchunks * info.elem_bytes * align16(info.chunk_bytes / info.elem_bytes);
  }
  *ws_nbytes = total;
  return LTC_OK;
}

int ltc_decompress_delta_batch(int count, const void* const* h_headers, const void* const* h_blob_ptrs,
                               const uint64_t* h_blob_nbytes, const void* const* h_base_ptrs,
                               void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                               int32_t* d_status, void* d_ws, uint64_t ws_nbytes, hipStream_t stream) {
  if (!h_base_ptrs) return LTC_ERR_INVALID_ARGUMENT;
  return decompress_impl(count, h_headers, h_blob_ptrs, h_blob_nbytes, h_dst_ptrs, h_dst_capacity,
                         d_status, stream, nullptr, nullptr, nullptr, h_base_ptrs, d_ws, ws_nbytes);
}

int ltc_decompress_delta(const void* h_header, const void* d_blob, uint64_t blob_nbytes,
                         const void* d_base, void* d_dst, uint64_t dst_capacity, int32_t* d_status,
                         void* d_ws, uint64_t ws_nbytes, hipStream_t stream) {
  return ltc_decompress_delta_batch(1, &h_header, &d_blob, &blob_nbytes, &d_base, &d_dst, &dst_capacity,
                                    d_status, d_ws, ws_nbytes, stream);
}

int ltc_decompress_batch_prof(int count, const void* const* h_headers, const void* const* h_blob_ptrs,
                              const uint64_t* h_blob_nbytes, void* const* h_dst_ptrs,
                              const uint64_t* h_dst_capacity, int32_t* d_status, hipStream_t stream,
                              const hipEvent_t* h_events) {
  return decompress_impl(count, h_headers, h_blob_ptrs, h_blob_nbytes, h_dst_ptrs, h_dst_capacity,
                         d_status, stream, h_events);
}

int ltc_decompress_from_host(const void* h_blob, uint64_t blob_nbytes, void* d_dst,
                             uint64_t dst_capacity, int32_t* d_status, void* d_stage,
                             uint64_t stage_capacity, hipStream_t stream) {
  return ltc_decompress_batch_from_host(1, &h_blob, &blob_nbytes, &d_dst, &dst_capacity, d_status,
                                        &d_stage, &stage_capacity, stream);
}

int ltc_decompress_batch_from_host(int count, const void* const* h_blobs, const uint64_t* h_blob_nbytes,
                                   void* const* h_dst_ptrs, const uint64_t* h_dst_capacity,
                                   int32_t* d_status, void* const* h_stage_ptrs,
                                   const uint64_t* h_stage_capacity, hipStream_t stream) {
  if (count < 1 || count > kMaxJobs || !h_blobs || !h_blob_nbytes || !h_stage_ptrs || !h_stage_capacity)
    return LTC_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < count; ++i) {
    if (!h_blobs[i]) return LTC_ERR_INVALID_ARGUMENT;
    if (h_blob_nbytes[i] < kHeader) return LTC_ERR_CORRUPT;
  }
  // the headers are the first bytes of the host blobs
  return decompress_impl(count, h_blobs, const_cast<const void* const*>(h_stage_ptrs), h_blob_nbytes,
                         h_dst_ptrs, h_dst_capacity, d_status, stream, nullptr, h_blobs,
                         h_stage_capacity);
}

int ltc_crc32_chunks_batch(int count, const void* const* h_src_ptrs, const uint64_t* h_nbytes,
                           uint32_t chunk_bytes, uint32_t* const* h_crc_ptrs, hipStream_t stream) {
  if (count < 1 || count > kMaxJobs || !h_src_ptrs || !h_nbytes || !h_crc_ptrs || chunk_bytes == 0)
    return LTC_ERR_INVALID_ARGUMENT;
  CrcArgs a;
  memset(&a, 0, sizeof(a));
  a.count = (uint32_t)count;
  a.chunk_bytes = chunk_bytes;
  a.seg = round_up(chunk_bytes, 256) / 64;
  for (int l = 0; l < 6; ++l) a.lvl[l] = xpow8(a.seg << l);
  uint64_t total = 0;
  for (int i = 0; i < count; ++i) {
    CrcJob& jb = a.jobs[i];
    jb.src = static_cast<const uint8_t*>(h_src_ptrs[i]);
    jb.out = h_crc_ptrs[i];
    jb.chunk0 = total;
    jb.nchunks = (h_nbytes[i] + chunk_bytes - 1) / chunk_bytes;
    if (jb.nchunks && (!jb.src || !jb.out)) return LTC_ERR_INVALID_ARGUMENT;
    jb.tail_len = jb.nchunks ? h_nbytes[i] - (jb.nchunks - 1) * (uint64_t)chunk_bytes : 0;
    total += jb.nchunks;
  }
  a.total_chunks = total;
  return launch_crc32(a, stream) == hipSuccess ? LTC_OK : LTC_ERR_HIP;
}

int ltc_crc32_chunks(const void* d_src, uint64_t nbytes, uint32_t chunk_bytes, uint32_t* d_crc,
                     hipStream_t stream) {
  if (chunk_bytes == 0) return LTC_ERR_INVALID_ARGUMENT;
  if (nbytes == 0) return LTC_OK;
  if (!d_src || !d_crc) return LTC_ERR_INVALID_ARGUMENT;
  return ltc_crc32_chunks_batch(1, &d_src, &nbytes, chunk_bytes, &d_crc, stream);
}

}  // extern "C"
