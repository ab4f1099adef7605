/*
 * ltc_oracle.c -- plain scalar reference for the lossless tensor codec.
 *
 * TEST INFRASTRUCTURE ONLY (see ltc_oracle.h for the format and the pages it
 * follows).  Deliberately simple: one element, one byte, one symbol at a
 * time, exact integer arithmetic, linear searches.  The only concession to
 * speed is an optional OpenMP loop over independent chunks, which does not
 * change any output byte.
 */
#include "ltc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define M_TOTAL 4096u
#define LANES 64
#define RANS_LOW 65536u
#define HDR_BYTES 64u
#define DIR_BYTES 16u
#define RANS_FIXED 272u /* 16-byte prefix + 64 u32 states */

static uint64_t align16(uint64_t v) { return (v + 15u) & ~(uint64_t)15u; }

/* Directory index of the t-th payload in blob order, for k chunks of e
 * streams: directory order, or with the top-last layout (ltc_oracle.h) the
 * k*(e-1) lower streams in directory order followed by the k top streams. */
static uint64_t placed(uint64_t t, uint64_t k, int e, int top_last) {
  if (!top_last || e == 1) return t;
  uint64_t lower = k * (uint64_t)(e - 1);
  if (t < lower) return t / (uint64_t)(e - 1) * (uint64_t)e + t % (uint64_t)(e - 1);
  return (t - lower) * (uint64_t)e + (uint64_t)(e - 1);
}

int ltco_elem_bytes(int dtype) {
  switch (dtype) {
    case 0: return 1;
    case 1: return 2;
    case 2: return 2;
    case 3: return 4;
    default: return 0;
  }
}

static int mantissa_bits(int dtype) {
  switch (dtype) {
    case 1: return 7;   /* bfloat16: 1 sign, 8 exponent, 7 mantissa */
    case 2: return 10;  /* IEEE half: 1 sign, 5 exponent, 10 mantissa */
    case 3: return 23;  /* IEEE single: 1 sign, 8 exponent, 23 mantissa */
    default: return -1;
  }
}

/* Exponent extraction (NOTE-241: ZipNN, "Method" item 1 and "Concepts"):
 * move the exponent field to the top of the word so that for BF16 and FP32
 * it fills the most significant byte; the sign goes directly below it. */
uint32_t ltco_reorder(int dtype, uint32_t x) {
  int wm = mantissa_bits(dtype);
  if (wm < 0) return x;
  int w = 8 * ltco_elem_bytes(dtype);
  int we = w - 1 - wm;
  uint32_t e = (x >> wm) & ((1u << we) - 1u);
  uint32_t s = (x >> (w - 1)) & 1u;
  uint32_t m = x & ((1u << wm) - 1u);
  return (e << (wm + 1)) | (s << wm) | m;
}

uint32_t ltco_unreorder(int dtype, uint32_t y) {
  int wm = mantissa_bits(dtype);
  if (wm < 0) return y;
  int w = 8 * ltco_elem_bytes(dtype);
  int we = w - 1 - wm;
  uint32_t e = (y >> (wm + 1)) & ((1u << we) - 1u);
  uint32_t s = (y >> wm) & 1u;
  uint32_t m = y & ((1u << wm) - 1u);
  return (s << (w - 1)) | (e << wm) | m;
}

static uint32_t load_le(const uint8_t* p, int e) {
  uint32_t x = 0;
  for (int i = 0; i < e; i++) x |= (uint32_t)p[i] << (8 * i);
  return x;
}

static void store_le(uint8_t* p, int e, uint32_t x) {
  for (int i = 0; i < e; i++) p[i] = (uint8_t)(x >> (8 * i));
}

static void put_u16(uint8_t* p, uint32_t v) { store_le(p, 2, v); }
static void put_u32(uint8_t* p, uint32_t v) { store_le(p, 4, v); }
static void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get_u16(const uint8_t* p) { return load_le(p, 2); }
static uint32_t get_u32(const uint8_t* p) { return load_le(p, 4); }
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
  return v;
}

/* Byte grouping (NOTE-241: ZipNN, "Method" item 2): stream k of a chunk is
 * byte k (little-endian position) of every reordered element. */
uint64_t ltco_chunk_stream(const uint8_t* src, uint64_t nbytes, int dtype,
                           uint32_t chunk_bytes, uint64_t c, int k, uint8_t* out) {
  int e = ltco_elem_bytes(dtype);
  uint64_t start = c * (uint64_t)chunk_bytes;
  uint64_t end = start + chunk_bytes;
  if (end > nbytes) end = nbytes;
  uint64_t n = (end - start) / (uint64_t)e;
  for (uint64_t t = 0; t < n; t++) {
    uint32_t y = ltco_reorder(dtype, load_le(src + start + t * e, e));
    out[t] = (uint8_t)(y >> (8 * k));
  }
  return n;
}

void ltco_histogram(const uint8_t* sym, uint64_t n, uint64_t h[256]) {
  for (int v = 0; v < 256; v++) h[v] = 0;
  for (uint64_t t = 0; t < n; t++) h[sym[t]] += 1;
}

/* Normalisation of a histogram to a 2^12 total (the pages fix only the
 * total; the rule is this format's reading, stated in ltc_oracle.h). */
int ltco_normalize(const uint64_t h[256], uint16_t f[256]) {
  uint64_t n = 0;
  int nonzero = 0;
  for (int v = 0; v < 256; v++) {
    n += h[v];
    if (h[v]) nonzero++;
  }
  if (nonzero < 2) return LTCO_ERR_INVALID_ARGUMENT;
  uint64_t g[256];
  uint64_t total = 0;
  for (int v = 0; v < 256; v++) {
    if (h[v] == 0) {
      g[v] = 0;
    } else {
      g[v] = h[v] * M_TOTAL / n;
      if (g[v] < 1) g[v] = 1;
    }
    total += g[v];
  }
  while (total > M_TOTAL) {
    int best = -1;
    for (int v = 0; v < 256; v++)
      if (g[v] > 1 && (best < 0 || g[v] > g[best])) best = v;
    g[best] -= 1;
    total -= 1;
  }
  if (total < M_TOTAL) {
    int best = 0;
    for (int v = 1; v < 256; v++)
      if (h[v] > h[best]) best = v;
    g[best] += M_TOTAL - total;
  }
  for (int v = 0; v < 256; v++) f[v] = (uint16_t)g[v];
  return LTCO_OK;
}

/* passthrough_threshold (cuZipNN 0.1.0, "API"): a stream stays coded only if
 * its payload is strictly below theta times its raw size, compared in IEEE
 * double.  Returns the largest integer P with (double)P < theta*(double)n. */
uint64_t ltco_p_max(uint64_t n, double theta) {
  double t = theta * (double)n;
  if (!(t > 0.0)) return 0;
  double p = floor(t);
  if (p >= t) p -= 1.0;
  if (p < 0.0) return 0;
  return (uint64_t)p;
}

static void cumulative(const uint16_t f[256], uint32_t cum[256]) {
  uint32_t acc = 0;
  for (int v = 0; v < 256; v++) {
    cum[v] = acc;
    acc += f[v];
  }
}

/* Interleaved rANS encoder (lmz README, "On a GPU": interleaved states are
 * lanes of work).  Walks the symbols in exactly the reverse of the decoder's
 * order and records each emitted word; the final list is reversed so that
 * it reads in decoder order. */
int ltco_rans_encode(const uint8_t* sym, uint64_t n, const uint16_t f[256],
                     uint32_t states[64], uint16_t* words, uint64_t words_cap,
                     uint64_t* nwords) {
  uint32_t cum[256];
  cumulative(f, cum);
  uint32_t x[LANES];
  for (int l = 0; l < LANES; l++) x[l] = RANS_LOW;
  uint64_t steps = (n + LANES - 1) / LANES;
  uint16_t* emitted = (uint16_t*)malloc((n ? n : 1) * sizeof(uint16_t));
  if (!emitted) return LTCO_ERR_INVALID_ARGUMENT;
  uint64_t count = 0;
  for (uint64_t j = steps; j-- > 0;) {
    for (int l = LANES - 1; l >= 0; l--) {
      uint64_t t = j * LANES + (uint64_t)l;
      if (t >= n) continue;
      uint32_t s = sym[t];
      uint32_t fs = f[s];
      if (fs == 0) {
        free(emitted);
        return LTCO_ERR_INVALID_ARGUMENT;
      }
      if ((uint64_t)x[l] >= ((uint64_t)fs << 20)) {
        emitted[count++] = (uint16_t)(x[l] & 0xFFFFu);
        x[l] >>= 16;
      }
      x[l] = (x[l] / fs) * M_TOTAL + (x[l] % fs) + cum[s];
    }
  }
  if (count > words_cap) {
    free(emitted);
    return LTCO_ERR_CAPACITY;
  }
  for (uint64_t i = 0; i < count; i++) words[i] = emitted[count - 1 - i];
  for (int l = 0; l < LANES; l++) states[l] = x[l];
  *nwords = count;
  free(emitted);
  return LTCO_OK;
}

int ltco_rans_decode(const uint16_t* words, uint64_t nwords,
                     const uint32_t states[64], const uint16_t f[256],
                     uint64_t n, uint8_t* out) {
  uint32_t cum[256];
  uint32_t total = 0;
  for (int v = 0; v < 256; v++) total += f[v];
  if (total != M_TOTAL) return LTCO_ERR_CORRUPT;
  cumulative(f, cum);
  uint32_t x[LANES];
  for (int l = 0; l < LANES; l++) x[l] = states[l];
  uint64_t steps = (n + LANES - 1) / LANES;
  uint64_t pos = 0;
  for (uint64_t j = 0; j < steps; j++) {
    for (int l = 0; l < LANES; l++) {
      uint64_t t = j * LANES + (uint64_t)l;
      if (t >= n) continue;
      uint32_t slot = x[l] & (M_TOTAL - 1u);
      int s = -1;
      for (int v = 0; v < 256; v++) {
        if (f[v] != 0 && cum[v] <= slot && slot < cum[v] + f[v]) {
          s = v;
          break;
        }
      }
      if (s < 0) return LTCO_ERR_CORRUPT;
      out[t] = (uint8_t)s;
      x[l] = f[s] * (x[l] >> 12) + slot - cum[s];
      if (x[l] < RANS_LOW) {
        if (pos >= nwords) return LTCO_ERR_CORRUPT;
        x[l] = (x[l] << 16) | words[pos];
        pos++;
      }
    }
  }
  if (pos != nwords) return LTCO_ERR_CORRUPT;
  for (int l = 0; l < LANES; l++)
    if (x[l] != RANS_LOW) return LTCO_ERR_CORRUPT;
  return LTCO_OK;
}

uint64_t ltco_compress_bound(uint64_t nbytes, int dtype, uint32_t chunk_bytes) {
  int e = ltco_elem_bytes(dtype);
  if (e == 0 || chunk_bytes == 0) return 0;
  uint64_t k = (nbytes + chunk_bytes - 1) / chunk_bytes;
  uint64_t bound = HDR_BYTES + DIR_BYTES * k * (uint64_t)e;
  for (uint64_t c = 0; c < k; c++) {
    uint64_t len = nbytes - c * (uint64_t)chunk_bytes;
    if (len > chunk_bytes) len = chunk_bytes;
    bound += (uint64_t)e * align16(len / (uint64_t)e);
  }
  return bound;
}

typedef struct {
  uint8_t mode;
  uint8_t cval;
  uint32_t size;
  uint8_t* payload; /* malloc'd, size bytes (NULL for CONST) */
} stream_result;

/* ---- deltas (NOTE-241: ZipNN, "Method" item 6 and "Key results", Deltas) --
 * ZipNN's rule picks a coder for runs of zeros over its order-0 coder when
 * more than 90% of a byte group is zero bytes or a zero run is longer than 3%
 * of it.  READING: the byte group is the chunk's stream, the run coder is the
 * ZRUN payload below, and the rule only admits ZRUN as a candidate: the
 * stream takes the smaller of RANS and ZRUN (ties: RANS), RAW if neither is
 * at most P_max. */
static int zrun_rule(const uint8_t* sym, uint64_t n) {
  uint64_t zeros = 0, run = 0, longest = 0;
  for (uint64_t i = 0; i < n; i++) {
    if (sym[i] == 0) {
      zeros++;
      run++;
      if (run > longest) longest = run;
    } else {
      run = 0;
    }
  }
  return 10 * zeros > 9 * n || 100 * longest > 3 * n;
}

/* ZRUN payload: u32 nnz | u32 nblk | 8 zero bytes | bitmap of the nonzero
 * 64-byte blocks (bit b = block b, least significant bit first), zero-padded
 * to 16 | one u64 per nonzero block (bit i = its byte i is nonzero), padded to
 * 16 | the nnz nonzero bytes in order. */
static uint64_t zrun_size(const uint8_t* sym, uint64_t n, uint64_t* nnz_out, uint64_t* nblk_out) {
  uint64_t nb = (n + 63) / 64, nnz = 0, nblk = 0;
  for (uint64_t b = 0; b < nb; b++) {
    int any = 0;
    for (uint64_t i = 64 * b; i < n && i < 64 * b + 64; i++)
      if (sym[i]) {
        any = 1;
        nnz++;
      }
    nblk += (uint64_t)any;
  }
  *nnz_out = nnz;
  *nblk_out = nblk;
  return 16 + align16((nb + 7) / 8) + align16(8 * nblk) + nnz;
}

static uint8_t* zrun_payload(const uint8_t* sym, uint64_t n, uint64_t size) {
  uint64_t nnz = 0, nblk = 0;
  zrun_size(sym, n, &nnz, &nblk);
  uint8_t* pl = (uint8_t*)calloc(size, 1);
  if (!pl) return NULL;
  uint64_t nb = (n + 63) / 64;
  uint64_t l2 = 16 + align16((nb + 7) / 8), lit = l2 + align16(8 * nblk);
  put_u32(pl, (uint32_t)nnz);
  put_u32(pl + 4, (uint32_t)nblk);
  uint64_t k = 0;
  for (uint64_t b = 0; b < nb; b++) {
    uint64_t mask = 0;
    for (uint64_t i = 64 * b; i < n && i < 64 * b + 64; i++)
      if (sym[i]) {
        mask |= 1ull << (i - 64 * b);
        pl[lit++] = sym[i];
      }
    if (mask) {
      pl[16 + b / 8] |= (uint8_t)(1u << (b % 8));
      put_u64(pl + l2 + 8 * k, mask);
      k++;
    }
  }
  return pl;
}

/* ZRUN payload -> the n stream bytes; checks every field */
static int zrun_decode(const uint8_t* pl, uint32_t size, uint64_t n, uint8_t* out) {
  if (size < 16) return LTCO_ERR_CORRUPT;
  uint64_t nnz = get_u32(pl), nblk = get_u32(pl + 4);
  for (int i = 8; i < 16; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  uint64_t nb = (n + 63) / 64;
  uint64_t l2 = 16 + align16((nb + 7) / 8), lit = l2 + align16(8 * nblk);
  if (nblk > nb || nnz > n || lit + nnz != size) return LTCO_ERR_CORRUPT;
  for (uint64_t i = 16 + (nb + 7) / 8; i < l2; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  if (nb % 8 && (pl[16 + nb / 8] >> (nb % 8))) return LTCO_ERR_CORRUPT;
  for (uint64_t i = l2 + 8 * nblk; i < lit; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  uint64_t k = 0, used = 0;
  for (uint64_t b = 0; b < nb; b++) {
    uint64_t mask = 0;
    if ((pl[16 + b / 8] >> (b % 8)) & 1) {
      if (k >= nblk) return LTCO_ERR_CORRUPT;
      mask = get_u64(pl + l2 + 8 * k);
      k++;
      if (mask == 0) return LTCO_ERR_CORRUPT;
    }
    for (uint64_t i = 64 * b; i < 64 * b + 64; i++) {
      const int nz = (int)((mask >> (i - 64 * b)) & 1);
      if (i >= n) {
        if (nz) return LTCO_ERR_CORRUPT;
        continue;
      }
      if (nz) {
        if (used >= nnz || pl[lit + used] == 0) return LTCO_ERR_CORRUPT;
        out[i] = pl[lit + used++];
      } else {
        out[i] = 0;
      }
    }
  }
  if (k != nblk || used != nnz) return LTCO_ERR_CORRUPT;
  return LTCO_OK;
}

/* a delta stream whose rule fires: ZRUN instead of RANS when strictly
 * smaller and at most P_max (p = the RANS payload size) */
static int maybe_zrun(const uint8_t* sym, uint64_t n, double theta, uint64_t p, stream_result* r) {
  if (!zrun_rule(sym, n)) return 0;
  uint64_t nnz = 0, nblk = 0;
  uint64_t pz = zrun_size(sym, n, &nnz, &nblk);
  if (pz >= p || pz > ltco_p_max(n, theta)) return 0;
  r->payload = zrun_payload(sym, n, pz);
  if (!r->payload) return -1;
  r->mode = LTCO_MODE_ZRUN;
  r->size = (uint32_t)pz;
  return 1;
}

/* One stream: histogram, CONST / RANS / RAW decision, payload bytes. */
static int encode_stream(const uint8_t* sym, uint64_t n, double theta,
                         stream_result* r, int delta) {
  uint64_t h[256];
  ltco_histogram(sym, n, h);
  int nonzero = 0, only = 0;
  for (int v = 0; v < 256; v++)
    if (h[v]) {
      nonzero++;
      only = v;
    }
  r->payload = NULL;
  r->cval = 0;
  if (nonzero == 1) {
    /* NOTE-241: ZipNN, "Method" item 3: a constant stream costs a header */
    r->mode = LTCO_MODE_CONST;
    r->cval = (uint8_t)only;
    r->size = 0;
    return LTCO_OK;
  }
  uint16_t f[256];
  int rc = ltco_normalize(h, f);
  if (rc) return rc;
  uint32_t states[64];
  uint16_t* words = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!words) return LTCO_ERR_INVALID_ARGUMENT;
  uint64_t nw = 0;
  rc = ltco_rans_encode(sym, n, f, states, words, n, &nw);
  if (rc) {
    free(words);
    return rc;
  }
  int lo = 0, hi = 255;
  while (h[lo] == 0) lo++;
  while (h[hi] == 0) hi--;
  uint64_t tcount = (uint64_t)(hi - lo + 1);
  uint64_t wo = align16(RANS_FIXED + 2 * tcount);
  uint64_t p = wo + 2 * nw;
  int z = delta ? maybe_zrun(sym, n, theta, p, r) : 0;
  if (z) {
    free(words);
    return z < 0 ? LTCO_ERR_INVALID_ARGUMENT : LTCO_OK;
  }
  if (p <= ltco_p_max(n, theta)) {
    uint8_t* pl = (uint8_t*)calloc(p, 1);
    if (!pl) {
      free(words);
      return LTCO_ERR_INVALID_ARGUMENT;
    }
    put_u32(pl + 0, (uint32_t)nw);
    pl[4] = (uint8_t)lo;
    pl[5] = (uint8_t)hi;
    for (int l = 0; l < LANES; l++) put_u32(pl + 16 + 4 * l, states[l]);
    for (uint64_t i = 0; i < tcount; i++) put_u16(pl + RANS_FIXED + 2 * i, f[lo + i]);
    for (uint64_t i = 0; i < nw; i++) put_u16(pl + wo + 2 * i, words[i]);
    r->mode = LTCO_MODE_RANS;
    r->size = (uint32_t)p;
    r->payload = pl;
  } else {
    /* cuZipNN 0.1.0, "API", passthrough_threshold: stored raw */
    uint8_t* pl = (uint8_t*)malloc(n);
    if (!pl) {
      free(words);
      return LTCO_ERR_INVALID_ARGUMENT;
    }
    memcpy(pl, sym, n);
    r->mode = LTCO_MODE_RAW;
    r->size = (uint32_t)n;
    r->payload = pl;
  }
  free(words);
  return LTCO_OK;
}

static int encode_chunk_streams(const uint8_t* src, uint64_t nbytes, int dtype,
                                uint32_t chunk_bytes, double theta, uint64_t c,
                                stream_result* out, int delta) {
  int e = ltco_elem_bytes(dtype);
  uint8_t* sym = (uint8_t*)malloc(chunk_bytes / (uint32_t)e + 1);
  if (!sym) return LTCO_ERR_INVALID_ARGUMENT;
  int rc = LTCO_OK;
  for (int k = 0; k < e && rc == LTCO_OK; k++) {
    uint64_t n = ltco_chunk_stream(src, nbytes, dtype, chunk_bytes, c, k, sym);
    rc = encode_stream(sym, n, theta, &out[k], delta);
  }
  free(sym);
  return rc;
}

static int check_args(uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                      double theta) {
  int e = ltco_elem_bytes(dtype);
  if (e == 0) return LTCO_ERR_UNSUPPORTED_DTYPE;
  if (nbytes % (uint64_t)e) return LTCO_ERR_INVALID_ARGUMENT;
  if (chunk_bytes < 8 || chunk_bytes > (1u << 24) || chunk_bytes % 8)
    return LTCO_ERR_INVALID_ARGUMENT;
  if (!(theta > 0.0 && theta <= 1.0)) return LTCO_ERR_INVALID_ARGUMENT;
  if (nbytes / chunk_bytes + (nbytes % chunk_bytes != 0) >= (1ull << 32))
    return LTCO_ERR_INVALID_ARGUMENT;
  return LTCO_OK;
}

int ltco_encode_chunk(const uint8_t* src, uint64_t nbytes, int dtype,
                      uint32_t chunk_bytes, double theta, uint64_t c,
                      uint8_t* modes, uint8_t* cvals, uint32_t* sizes,
                      uint8_t* out, uint64_t out_cap, uint64_t* nout) {
  int rc = check_args(nbytes, dtype, chunk_bytes, theta);
  if (rc) return rc;
  int e = ltco_elem_bytes(dtype);
  if (c * (uint64_t)chunk_bytes >= nbytes) return LTCO_ERR_INVALID_ARGUMENT;
  stream_result r[4];
  memset(r, 0, sizeof(r));
  rc = encode_chunk_streams(src, nbytes, dtype, chunk_bytes, theta, c, r, 0);
  uint64_t cur = 0;
  for (int k = 0; k < e && rc == LTCO_OK; k++) {
    uint64_t next = align16(cur + r[k].size);
    if (next > out_cap) {
      rc = LTCO_ERR_CAPACITY;
      break;
    }
    if (r[k].size) memcpy(out + cur, r[k].payload, r[k].size);
    memset(out + cur + r[k].size, 0, next - cur - r[k].size);
    modes[k] = r[k].mode;
    cvals[k] = r[k].cval;
    sizes[k] = r[k].size;
    cur = next;
  }
  for (int k = 0; k < e; k++) free(r[k].payload);
  *nout = cur;
  return rc;
}

static int compress_v1(const uint8_t* src, uint64_t nbytes, int dtype,
                       uint32_t chunk_bytes, double theta, uint8_t* blob,
                       uint64_t blob_capacity, uint64_t* blob_nbytes, int nthreads,
                       int delta, int top_last) {
  int rc = LTCO_OK;
  int e = ltco_elem_bytes(dtype);
  uint64_t k = (nbytes + chunk_bytes - 1) / chunk_bytes;
  uint64_t s = k * (uint64_t)e;
  stream_result* res = (stream_result*)calloc(s ? s : 1, sizeof(stream_result));
  if (!res) return LTCO_ERR_INVALID_ARGUMENT;
  int failed = 0;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long long c = 0; c < (long long)k; c++) {
    int r = encode_chunk_streams(src, nbytes, dtype, chunk_bytes, theta,
                                 (uint64_t)c, res + (uint64_t)c * e, delta);
    if (r) {
#pragma omp atomic write
      failed = r;
    }
  }
  uint64_t base = HDR_BYTES + DIR_BYTES * s;
  uint64_t cursor = base;
  for (uint64_t i = 0; i < s; i++) cursor = align16(cursor + res[i].size);
  if (failed) {
    rc = failed;
  } else if (cursor > blob_capacity) {
    rc = LTCO_ERR_CAPACITY;
  } else {
    memset(blob, 0, cursor);
    memcpy(blob, "LTCB", 4);
    put_u16(blob + 4, 1);
    blob[6] = (uint8_t)dtype;
    blob[7] = (uint8_t)e;
    put_u64(blob + 8, nbytes);
    put_u32(blob + 16, chunk_bytes);
    put_u32(blob + 20, (uint32_t)k);
    put_u16(blob + 24, LANES);
    blob[26] = 12;
    blob[27] = (uint8_t)((delta ? LTCO_FLAG_DELTA : 0) | (top_last ? LTCO_FLAG_TOP_LAST : 0));
    put_u64(blob + 32, cursor);
    put_u64(blob + 40, base);
    uint64_t cur = base;
    for (uint64_t t = 0; t < s; t++) {
      uint64_t i = placed(t, k, e, top_last);
      uint8_t* d = blob + HDR_BYTES + DIR_BYTES * i;
      put_u64(d, cur);
      put_u32(d + 8, res[i].size);
      d[12] = res[i].mode;
      d[13] = res[i].cval;
      if (res[i].size) memcpy(blob + cur, res[i].payload, res[i].size);
      cur = align16(cur + res[i].size);
    }
    *blob_nbytes = cursor;
  }
  for (uint64_t i = 0; i < s; i++) free(res[i].payload);
  free(res);
  return rc;
}

int ltco_compress(const uint8_t* src, uint64_t nbytes, int dtype,
                  uint32_t chunk_bytes, double theta, uint8_t* blob,
                  uint64_t blob_capacity, uint64_t* blob_nbytes, int nthreads) {
  int rc = check_args(nbytes, dtype, chunk_bytes, theta);
  if (rc) return rc;
  return compress_v1(src, nbytes, dtype, chunk_bytes, theta, blob, blob_capacity, blob_nbytes,
                     nthreads, 0, 0);
}

/* ---- format v2: one frequency table per stream index (shared tables) ---- */

/* bytes of a table record: 16-byte head plus f[lo..hi], padded to 16 */
static uint64_t record_bytes(int lo, int hi) {
  return lo > hi ? 16u : align16(16u + 2u * (uint64_t)(hi - lo + 1));
}

/* v2 stream: CONST as in v1; otherwise coded with the plane's table f (which
 * covers every value of the stream) and kept if the payload (272 + 2W bytes)
 * is at most P_max, else RAW. */
static int encode_stream_shared(const uint8_t* sym, uint64_t n, double theta,
                                const uint16_t f[256], stream_result* r, int delta) {
  uint64_t h[256];
  ltco_histogram(sym, n, h);
  int nonzero = 0, only = 0;
  for (int v = 0; v < 256; v++)
    if (h[v]) {
      nonzero++;
      only = v;
    }
  r->payload = NULL;
  r->cval = 0;
  if (nonzero == 1) {
    r->mode = LTCO_MODE_CONST;
    r->cval = (uint8_t)only;
    r->size = 0;
    return LTCO_OK;
  }
  uint32_t states[64];
  uint16_t* words = (uint16_t*)malloc(n * sizeof(uint16_t));
  if (!words) return LTCO_ERR_INVALID_ARGUMENT;
  uint64_t nw = 0;
  int rc = ltco_rans_encode(sym, n, f, states, words, n, &nw);
  if (rc) {
    free(words);
    return rc;
  }
  uint64_t p = RANS_FIXED + 2 * nw;
  int z = delta ? maybe_zrun(sym, n, theta, p, r) : 0;
  if (z) {
    free(words);
    return z < 0 ? LTCO_ERR_INVALID_ARGUMENT : LTCO_OK;
  }
  if (p <= ltco_p_max(n, theta)) {
    uint8_t* pl = (uint8_t*)calloc(p, 1);
    if (!pl) {
      free(words);
      return LTCO_ERR_INVALID_ARGUMENT;
    }
    put_u32(pl + 0, (uint32_t)nw);
    for (int l = 0; l < LANES; l++) put_u32(pl + 16 + 4 * l, states[l]);
    for (uint64_t i = 0; i < nw; i++) put_u16(pl + RANS_FIXED + 2 * i, words[i]);
    r->mode = LTCO_MODE_RANS;
    r->size = (uint32_t)p;
    r->payload = pl;
  } else {
    uint8_t* pl = (uint8_t*)malloc(n);
    if (!pl) {
      free(words);
      return LTCO_ERR_INVALID_ARGUMENT;
    }
    memcpy(pl, sym, n);
    r->mode = LTCO_MODE_RAW;
    r->size = (uint32_t)n;
    r->payload = pl;
  }
  free(words);
  return LTCO_OK;
}

uint64_t ltco_compress_bound_ex(uint64_t nbytes, int dtype, uint32_t chunk_bytes,
                                uint32_t flags) {
  uint64_t b = ltco_compress_bound(nbytes, dtype, chunk_bytes);
  if (b && (flags & LTCO_FLAG_SHARED_TABLES))
    b += (uint64_t)ltco_elem_bytes(dtype) * record_bytes(0, 255);
  return b;
}

static int compress_shared(const uint8_t* src, uint64_t nbytes, int dtype,
                           uint32_t chunk_bytes, double theta, uint8_t* blob,
                           uint64_t blob_capacity, uint64_t* blob_nbytes,
                           int nthreads, int delta, int top_last) {
  int e = ltco_elem_bytes(dtype);
  uint64_t k = (nbytes + chunk_bytes - 1) / chunk_bytes;
  uint64_t s = k * (uint64_t)e;
  if (nthreads < 1) nthreads = 1;
  /* plane k's histogram: the sum of stream k's histograms over all chunks */
  uint64_t plane[4][256];
  memset(plane, 0, sizeof(plane));
  uint8_t* sym = (uint8_t*)malloc(chunk_bytes / (uint32_t)e + 1);
  if (!sym) return LTCO_ERR_INVALID_ARGUMENT;
  for (uint64_t c = 0; c < k; c++)
    for (int q = 0; q < e; q++) {
      uint64_t n = ltco_chunk_stream(src, nbytes, dtype, chunk_bytes, c, q, sym);
      uint64_t h[256];
      ltco_histogram(sym, n, h);
      for (int v = 0; v < 256; v++) plane[q][v] += h[v];
    }
  free(sym);
  uint16_t f[4][256];
  int lo[4], hi[4];
  for (int q = 0; q < e; q++) {
    lo[q] = 0;
    hi[q] = 255;
    while (lo[q] < 256 && plane[q][lo[q]] == 0) lo[q]++;
    while (hi[q] >= 0 && plane[q][hi[q]] == 0) hi[q]--;
    memset(f[q], 0, sizeof(f[q]));
    if (lo[q] < hi[q]) {
      int rc = ltco_normalize(plane[q], f[q]);
      if (rc) return rc;
    } else {  /* at most one value in the whole plane: no table */
      lo[q] = 1;
      hi[q] = 0;
    }
  }
  stream_result* res = (stream_result*)calloc(s ? s : 1, sizeof(stream_result));
  if (!res) return LTCO_ERR_INVALID_ARGUMENT;
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long long c = 0; c < (long long)k; c++) {
    uint8_t* cs = (uint8_t*)malloc(chunk_bytes / (uint32_t)e + 1);
    int r = cs ? LTCO_OK : LTCO_ERR_INVALID_ARGUMENT;
    for (int q = 0; q < e && r == LTCO_OK; q++) {
      uint64_t n = ltco_chunk_stream(src, nbytes, dtype, chunk_bytes, (uint64_t)c, q, cs);
      r = encode_stream_shared(cs, n, theta, f[q], res + (uint64_t)c * e + q, delta);
    }
    free(cs);
    if (r) {
#pragma omp atomic write
      failed = r;
    }
  }
  uint64_t tables = 0;
  for (int q = 0; q < e; q++) tables += record_bytes(lo[q], hi[q]);
  uint64_t base = HDR_BYTES + DIR_BYTES * s + tables;
  uint64_t cursor = base;
  for (uint64_t i = 0; i < s; i++) cursor = align16(cursor + res[i].size);
  int rc = LTCO_OK;
  if (failed) {
    rc = failed;
  } else if (cursor > blob_capacity) {
    rc = LTCO_ERR_CAPACITY;
  } else {
    memset(blob, 0, cursor);
    memcpy(blob, "LTCB", 4);
    put_u16(blob + 4, 2);
    blob[6] = (uint8_t)dtype;
    blob[7] = (uint8_t)e;
    put_u64(blob + 8, nbytes);
    put_u32(blob + 16, chunk_bytes);
    put_u32(blob + 20, (uint32_t)k);
    put_u16(blob + 24, LANES);
    blob[26] = 12;
    blob[27] = (uint8_t)(LTCO_FLAG_SHARED_TABLES | (delta ? LTCO_FLAG_DELTA : 0) |
                         (top_last ? LTCO_FLAG_TOP_LAST : 0));
    put_u64(blob + 32, cursor);
    put_u64(blob + 40, base);
    uint64_t t = HDR_BYTES + DIR_BYTES * s;
    for (int q = 0; q < e; q++) {
      put_u16(blob + t, (uint32_t)lo[q]);
      put_u16(blob + t + 2, (uint32_t)hi[q]);
      for (int v = lo[q]; v <= hi[q]; v++) put_u16(blob + t + 16 + 2 * (uint64_t)(v - lo[q]), f[q][v]);
      t += record_bytes(lo[q], hi[q]);
    }
    uint64_t cur = base;
    for (uint64_t t = 0; t < s; t++) {
      uint64_t i = placed(t, k, e, top_last);
      uint8_t* d = blob + HDR_BYTES + DIR_BYTES * i;
      put_u64(d, cur);
      put_u32(d + 8, res[i].size);
      d[12] = res[i].mode;
      d[13] = res[i].cval;
      if (res[i].size) memcpy(blob + cur, res[i].payload, res[i].size);
      cur = align16(cur + res[i].size);
    }
    *blob_nbytes = cursor;
  }
  for (uint64_t i = 0; i < s; i++) free(res[i].payload);
  free(res);
  return rc;
}

int ltco_compress_ex(const uint8_t* src, uint64_t nbytes, int dtype,
                     uint32_t chunk_bytes, double theta, uint32_t flags,
                     uint8_t* blob, uint64_t blob_capacity, uint64_t* blob_nbytes,
                     int nthreads) {
  if (flags & ~(uint32_t)(LTCO_FLAG_SHARED_TABLES | LTCO_FLAG_TOP_LAST))
    return LTCO_ERR_INVALID_ARGUMENT;
  int rc = check_args(nbytes, dtype, chunk_bytes, theta);
  if (rc) return rc;
  int top_last = (flags & LTCO_FLAG_TOP_LAST) != 0;
  if (!(flags & LTCO_FLAG_SHARED_TABLES))
    return compress_v1(src, nbytes, dtype, chunk_bytes, theta, blob, blob_capacity, blob_nbytes,
                       nthreads, 0, top_last);
  return compress_shared(src, nbytes, dtype, chunk_bytes, theta, blob, blob_capacity,
                         blob_nbytes, nthreads, 0, top_last);
}

int ltco_compress_delta(const uint8_t* src, const uint8_t* base, uint64_t nbytes, int dtype,
                        uint32_t chunk_bytes, double theta, uint32_t flags, uint8_t* blob,
                        uint64_t blob_capacity, uint64_t* blob_nbytes, int nthreads) {
  if (flags & ~(uint32_t)(LTCO_FLAG_SHARED_TABLES | LTCO_FLAG_TOP_LAST))
    return LTCO_ERR_INVALID_ARGUMENT;
  int rc = check_args(nbytes, dtype, chunk_bytes, theta);
  if (rc) return rc;
  int top_last = (flags & LTCO_FLAG_TOP_LAST) != 0;
  /* NOTE-241: ZipNN, "Method" item 6: XOR against the base, then as usual */
  uint8_t* x = (uint8_t*)malloc(nbytes ? nbytes : 1);
  if (!x) return LTCO_ERR_INVALID_ARGUMENT;
  for (uint64_t i = 0; i < nbytes; i++) x[i] = src[i] ^ base[i];
  if (flags & LTCO_FLAG_SHARED_TABLES)
    rc = compress_shared(x, nbytes, dtype, chunk_bytes, theta, blob, blob_capacity, blob_nbytes,
                         nthreads, 1, top_last);
  else
    rc = compress_v1(x, nbytes, dtype, chunk_bytes, theta, blob, blob_capacity, blob_nbytes,
                     nthreads, 1, top_last);
  free(x);
  return rc;
}

typedef struct {
  uint64_t off;
  uint32_t size;
  uint8_t mode;
  uint8_t cval;
} dir_entry;

/* a v2 blob's tables, one per stream index (present = 0: no table) */
typedef struct {
  int present[4];
  uint16_t f[4][256];
} shared_tables;

/* Structural checks of one RANS payload (lo, hi, zeros, table, states). */
static int check_rans_payload(const uint8_t* pl, uint32_t size, uint16_t f[256],
                              uint32_t states[64], uint64_t* nwords,
                              uint64_t* words_off) {
  if (size < RANS_FIXED + 16u) return LTCO_ERR_CORRUPT;
  uint32_t nw = get_u32(pl);
  int lo = pl[4], hi = pl[5];
  if (lo >= hi) return LTCO_ERR_CORRUPT;
  for (int i = 6; i < 16; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  uint64_t tcount = (uint64_t)(hi - lo + 1);
  uint64_t wo = align16(RANS_FIXED + 2 * tcount);
  if (wo > size) return LTCO_ERR_CORRUPT;
  if ((uint64_t)size - wo != 2 * (uint64_t)nw) return LTCO_ERR_CORRUPT;
  for (uint64_t i = RANS_FIXED + 2 * tcount; i < wo; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  memset(f, 0, 256 * sizeof(uint16_t));
  uint32_t total = 0;
  for (uint64_t i = 0; i < tcount; i++) {
    f[lo + i] = (uint16_t)get_u16(pl + RANS_FIXED + 2 * i);
    total += f[lo + i];
  }
  if (f[lo] == 0 || f[hi] == 0 || total != M_TOTAL) return LTCO_ERR_CORRUPT;
  for (int l = 0; l < LANES; l++) {
    states[l] = get_u32(pl + 16 + 4 * l);
    if (states[l] < RANS_LOW) return LTCO_ERR_CORRUPT;
  }
  *nwords = nw;
  *words_off = wo;
  return LTCO_OK;
}

/* Structural checks of one v2 RANS payload (zeros, word count, states). */
static int check_shared_payload(const uint8_t* pl, uint32_t size, uint32_t states[64],
                                uint64_t* nwords) {
  if (size < RANS_FIXED) return LTCO_ERR_CORRUPT;
  uint32_t nw = get_u32(pl);
  for (int i = 4; i < 16; i++)
    if (pl[i]) return LTCO_ERR_CORRUPT;
  if ((uint64_t)size - RANS_FIXED != 2 * (uint64_t)nw) return LTCO_ERR_CORRUPT;
  for (int l = 0; l < LANES; l++) {
    states[l] = get_u32(pl + 16 + 4 * l);
    if (states[l] < RANS_LOW) return LTCO_ERR_CORRUPT;
  }
  *nwords = nw;
  return LTCO_OK;
}

static int decode_chunk(const uint8_t* blob, const dir_entry* ent, int dtype,
                        int e, uint64_t n, uint8_t* dst, const shared_tables* st) {
  uint8_t* planes = (uint8_t*)malloc((uint64_t)e * (n ? n : 1));
  if (!planes) return LTCO_ERR_INVALID_ARGUMENT;
  int rc = LTCO_OK;
  for (int k = 0; k < e && rc == LTCO_OK; k++) {
    uint8_t* plane = planes + (uint64_t)k * n;
    const uint8_t* pl = blob + ent[k].off;
    if (ent[k].mode == LTCO_MODE_CONST) {
      memset(plane, ent[k].cval, n);
    } else if (ent[k].mode == LTCO_MODE_RAW) {
      memcpy(plane, pl, n);
    } else if (ent[k].mode == LTCO_MODE_ZRUN) {
      rc = zrun_decode(pl, ent[k].size, n, plane);
    } else {
      uint16_t f[256];
      uint32_t states[64];
      uint64_t nw = 0, wo = 0;
      if (st) {  /* v2: the plane's table */
        if (!st->present[k]) {
          rc = LTCO_ERR_CORRUPT;
          break;
        }
        memcpy(f, st->f[k], sizeof(f));
        wo = RANS_FIXED;
        rc = check_shared_payload(pl, ent[k].size, states, &nw);
      } else {
        rc = check_rans_payload(pl, ent[k].size, f, states, &nw, &wo);
      }
      if (rc) break;
      uint16_t* words = (uint16_t*)malloc((nw ? nw : 1) * sizeof(uint16_t));
      if (!words) {
        rc = LTCO_ERR_INVALID_ARGUMENT;
        break;
      }
      for (uint64_t i = 0; i < nw; i++) words[i] = (uint16_t)get_u16(pl + wo + 2 * i);
      rc = ltco_rans_decode(words, nw, states, f, n, plane);
      free(words);
    }
  }
  if (rc == LTCO_OK) {
    for (uint64_t t = 0; t < n; t++) {
      uint32_t y = 0;
      for (int k = 0; k < e; k++) y |= (uint32_t)planes[(uint64_t)k * n + t] << (8 * k);
      store_le(dst + t * e, e, ltco_unreorder(dtype, y));
    }
  }
  free(planes);
  return rc;
}

/* base: the delta base (delta blobs only; NULL otherwise) */
static int decompress_impl(const uint8_t* blob, uint64_t blob_nbytes, const uint8_t* xbase,
                           uint8_t* dst, uint64_t dst_capacity, uint64_t* out_nbytes,
                           int nthreads) {
  if (blob_nbytes < HDR_BYTES) return LTCO_ERR_CORRUPT;
  if (memcmp(blob, "LTCB", 4) != 0) return LTCO_ERR_BAD_MAGIC;
  const int version = (int)get_u16(blob + 4);
  if (version != 1 && version != 2) return LTCO_ERR_BAD_VERSION;
  int dtype = blob[6];
  int e = ltco_elem_bytes(dtype);
  if (e == 0) return LTCO_ERR_UNSUPPORTED_DTYPE;
  if (blob[7] != e) return LTCO_ERR_CORRUPT;
  uint64_t nbytes = get_u64(blob + 8);
  uint32_t chunk_bytes = get_u32(blob + 16);
  uint64_t k = get_u32(blob + 20);
  const int delta = (blob[27] & LTCO_FLAG_DELTA) != 0;
  const int top_last = (blob[27] & LTCO_FLAG_TOP_LAST) != 0;
  if (get_u16(blob + 24) != LANES || blob[26] != 12 ||
      (blob[27] & ~(LTCO_FLAG_DELTA | LTCO_FLAG_TOP_LAST)) !=
          (version == 2 ? LTCO_FLAG_SHARED_TABLES : 0) ||
      get_u32(blob + 28) != 0)
    return LTCO_ERR_CORRUPT;
  if (delta != (xbase != NULL)) return LTCO_ERR_INVALID_ARGUMENT; /* a delta blob needs its base */
  for (int i = 48; i < 64; i++)
    if (blob[i]) return LTCO_ERR_CORRUPT;
  if (chunk_bytes < 8 || chunk_bytes > (1u << 24) || chunk_bytes % 8)
    return LTCO_ERR_CORRUPT;
  if (nbytes % (uint64_t)e) return LTCO_ERR_CORRUPT;
  /* K = ceil(N / C) as an exact integer (no wrap for N near 2^64) */
  if (k != nbytes / chunk_bytes + (nbytes % chunk_bytes != 0)) return LTCO_ERR_CORRUPT;
  uint64_t s = k * (uint64_t)e;
  uint64_t base = HDR_BYTES + DIR_BYTES * s;
  if (get_u64(blob + 32) != blob_nbytes) return LTCO_ERR_CORRUPT;
  if (base > blob_nbytes) return LTCO_ERR_CORRUPT;
  shared_tables st;
  if (version == 2) {
    /* table records follow the directory, one per stream index */
    uint64_t t = base;
    for (int q = 0; q < e; q++) {
      if (t + 16 > blob_nbytes) return LTCO_ERR_CORRUPT;
      int lo = (int)get_u16(blob + t), hi = (int)get_u16(blob + t + 2);
      for (int i = 4; i < 16; i++)
        if (blob[t + i]) return LTCO_ERR_CORRUPT;
      if (lo == 1 && hi == 0) {
        st.present[q] = 0;
        t += 16;
        continue;
      }
      if (lo >= hi || hi > 255) return LTCO_ERR_CORRUPT;
      uint64_t rb = record_bytes(lo, hi);
      if (t + rb > blob_nbytes) return LTCO_ERR_CORRUPT;
      memset(st.f[q], 0, sizeof(st.f[q]));
      uint32_t total = 0;
      for (int v = lo; v <= hi; v++) {
        st.f[q][v] = (uint16_t)get_u16(blob + t + 16 + 2 * (uint64_t)(v - lo));
        total += st.f[q][v];
      }
      for (uint64_t i = 16 + 2 * (uint64_t)(hi - lo + 1); i < rb; i++)
        if (blob[t + i]) return LTCO_ERR_CORRUPT;
      if (st.f[q][lo] == 0 || st.f[q][hi] == 0 || total != M_TOTAL) return LTCO_ERR_CORRUPT;
      st.present[q] = 1;
      t += rb;
    }
    base = t;
  }
  if (get_u64(blob + 40) != base) return LTCO_ERR_CORRUPT;
  if (dst_capacity < nbytes) return LTCO_ERR_CAPACITY;

  dir_entry* ent = (dir_entry*)malloc((s ? s : 1) * sizeof(dir_entry));
  if (!ent) return LTCO_ERR_INVALID_ARGUMENT;
  for (uint64_t i = 0; i < s; i++) {
    const uint8_t* d = blob + HDR_BYTES + DIR_BYTES * i;
    ent[i].off = get_u64(d);
    ent[i].size = get_u32(d + 8);
    ent[i].mode = d[12];
    ent[i].cval = d[13];
    uint64_t c = i / (uint64_t)e;
    uint64_t len = nbytes - c * (uint64_t)chunk_bytes;
    if (len > chunk_bytes) len = chunk_bytes;
    uint64_t n = len / (uint64_t)e;
    int bad = get_u16(d + 14) != 0 ||
              ent[i].mode > (delta ? LTCO_MODE_ZRUN : LTCO_MODE_CONST) ||
              (ent[i].mode != LTCO_MODE_CONST && ent[i].cval != 0) ||
              (ent[i].mode == LTCO_MODE_RAW && ent[i].size != n) ||
              (ent[i].mode == LTCO_MODE_CONST && ent[i].size != 0) ||
              ent[i].off > blob_nbytes || ent[i].size > blob_nbytes - ent[i].off;
    if (bad) {
      free(ent);
      return LTCO_ERR_CORRUPT;
    }
  }
  /* the offsets: each payload starts where the one before it in blob order
     ends (rounded up to 16), the first at payload_base, the last ends the blob */
  uint64_t cursor = base;
  for (uint64_t t = 0; t < s; t++) {
    uint64_t i = placed(t, k, e, top_last);
    if (ent[i].off != cursor) {
      free(ent);
      return LTCO_ERR_CORRUPT;
    }
    cursor = align16(ent[i].off + ent[i].size);
  }
  if (cursor != blob_nbytes) {
    free(ent);
    return LTCO_ERR_CORRUPT;
  }
  int failed = 0;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
  for (long long c = 0; c < (long long)k; c++) {
    uint64_t start = (uint64_t)c * chunk_bytes;
    uint64_t len = nbytes - start;
    if (len > chunk_bytes) len = chunk_bytes;
    int r = decode_chunk(blob, ent + (uint64_t)c * e, dtype, e, len / (uint64_t)e,
                         dst + start, version == 2 ? &st : NULL);
    if (r) {
#pragma omp atomic write
      failed = r;
    }
  }
  free(ent);
  if (failed) return failed;
  if (xbase)
    for (uint64_t i = 0; i < nbytes; i++) dst[i] ^= xbase[i];
  *out_nbytes = nbytes;
  return LTCO_OK;
}

int ltco_decompress(const uint8_t* blob, uint64_t blob_nbytes, uint8_t* dst,
                    uint64_t dst_capacity, uint64_t* out_nbytes, int nthreads) {
  return decompress_impl(blob, blob_nbytes, NULL, dst, dst_capacity, out_nbytes, nthreads);
}

int ltco_decompress_delta(const uint8_t* blob, uint64_t blob_nbytes, const uint8_t* base,
                          uint8_t* dst, uint64_t dst_capacity, uint64_t* out_nbytes,
                          int nthreads) {
  if (!base) return LTCO_ERR_INVALID_ARGUMENT;
  return decompress_impl(blob, blob_nbytes, base, dst, dst_capacity, out_nbytes, nthreads);
}

/* CRC-32 as zlib computes it (cuZipNN 0.1.0, "API": checksums match
 * zlib.crc32): reflected polynomial 0xEDB88320, one bit at a time. */
uint32_t ltco_crc32(const uint8_t* p, uint64_t n) {
  uint32_t c = 0xFFFFFFFFu;
  for (uint64_t i = 0; i < n; i++) {
    c ^= p[i];
    for (int b = 0; b < 8; b++) c = (c >> 1) ^ (0xEDB88320u & (0u - (c & 1u)));
  }
  return c ^ 0xFFFFFFFFu;
}

int ltco_crc32_chunks(const uint8_t* p, uint64_t n, uint32_t chunk_bytes,
                      uint32_t* out) {
  if (chunk_bytes == 0) return LTCO_ERR_INVALID_ARGUMENT;
  uint64_t count = (n + chunk_bytes - 1) / chunk_bytes;
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)count; i++) {
    uint64_t start = (uint64_t)i * chunk_bytes;
    uint64_t len = n - start;
    if (len > chunk_bytes) len = chunk_bytes;
    out[i] = ltco_crc32(p + start, len);
  }
  return LTCO_OK;
}
