// Fuzz driver for the library's host-side blob parsing (csrc/ltc_host.cpp),
// built by tests/test_host_sanitized.py with -fsanitize=address,undefined.
//
// For every blob file given on the command line it runs ltc_blob_info,
// ltc_blob_stats and the host-blob copy groups (as ltc_decompress_from_host
// would, when the header passes and its blob size matches) on the blob and
// on deterministic mutations of it: every truncation of the header and the
// directory, single-bit flips and random byte runs over the header and the
// directory, and extreme values in each header field.  Every buffer is a
// heap allocation of exactly its length, so a read past it is an ASan error.
// It also checks that every copy range lies inside its blob.  Prints one
// summary line; any sanitizer report or failed check exits non-zero.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "ltc.h"
#include "ltc_host.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_rand() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}

long g_runs = 0, g_ok_headers = 0, g_ranges = 0;
int g_fail = 0;

void fail(const char* what, uint64_t a, uint64_t b) {
  fprintf(stderr, "FAIL %s (%llu, %llu)\n", what, (unsigned long long)a, (unsigned long long)b);
  g_fail = 1;
}

// Everything the library's host code does with blob bytes, on a copy of
// `len` bytes that is its own heap allocation.
void exercise(const uint8_t* src, uint64_t len) {
  ++g_runs;
  uint8_t* p = static_cast<uint8_t*>(malloc(len ? len : 1));
  if (len) memcpy(p, src, len);
  ltc_info info;
  const int rc = ltc_blob_info(p, len, &info);
  ltc_stats st;
  (void)ltc_blob_stats(p, len, &st);
  if (rc == LTC_OK) {
    ++g_ok_headers;
    if (info.payload_base > info.blob_nbytes || info.elem_bytes == 0) fail("info fields", info.payload_base, info.blob_nbytes);
    // the prefix a caller passes to ltc_blob_stats: exactly payload_base bytes
    if (info.payload_base <= len) {
      uint8_t* q = static_cast<uint8_t*>(malloc(info.payload_base));
      memcpy(q, p, info.payload_base);
      (void)ltc_blob_stats(q, info.payload_base, &st);
      free(q);
    }
    // the host-blob decode runs only when the header's size is the buffer's
    if (info.blob_nbytes == len && info.nchunks > 0) {
      ltc::HostBlob hb[3];
      uint64_t chunk0 = 0, total = 0;
      for (int j = 0; j < 3; ++j) {  // three copies of the blob in one call
        hb[j] = ltc::HostBlob{p, len, chunk0, info.nchunks, (info.flags & LTC_FLAG_TOP_LAST) != 0};
        chunk0 += info.nchunks;
        total += len;
      }
      ltc::HostRange rg[6];
      for (uint64_t gb : {1ull << 10, 1ull << 20, 16ull << 20}) {
        const uint64_t G = ltc::host_copy_groups(total, chunk0, gb, 8);
        if (G < 1 || G > 8 || G > chunk0) fail("group count", G, chunk0);
        for (uint64_t g = 0; g < G; ++g) {
          const uint32_t n = ltc::host_group_ranges(hb, 3, info.elem_bytes, chunk0, G, g, rg);
          if (n > 6) fail("range count", n, g);
          for (uint32_t q = 0; q < n; ++q) {
            ++g_ranges;
            if (rg[q].job >= 3 || rg[q].lo >= rg[q].hi || rg[q].hi > len) fail("range", rg[q].lo, rg[q].hi);
          }
        }
      }
    }
  }
  free(p);
}

void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
void put16(uint8_t* p, uint16_t v) { memcpy(p, &v, 2); }

void fuzz_blob(const std::vector<uint8_t>& blob) {
  const uint64_t len = blob.size();
  exercise(blob.data(), len);
  ltc_info info;
  uint64_t meta = len < 64 ? len : 64;  // header, plus the directory when the header parses
  if (len >= 64 && ltc_blob_info(blob.data(), len, &info) == LTC_OK) meta = info.payload_base;
  // truncations: every length over the header and directory (capped), then random ones
  const uint64_t tmax = meta + 64 < len ? meta + 64 : len;
  for (uint64_t t = 0; t <= tmax && t <= 4096; ++t) exercise(blob.data(), t);
  for (int i = 0; i < 200 && len; ++i) exercise(blob.data(), next_rand() % len);
  std::vector<uint8_t> m;
  // single-bit flips in the header and directory
  for (int i = 0; i < 3000 && meta; ++i) {
    m = blob;
    const uint64_t bit = next_rand() % (8 * meta);
    m[bit / 8] ^= (uint8_t)(1u << (bit % 8));
    exercise(m.data(), len);
  }
  // random byte runs in the directory (the header kept, so it still parses)
  for (int i = 0; i < 2000 && meta > 64; ++i) {
    m = blob;
    const uint64_t at = 64 + next_rand() % (meta - 64);
    const uint64_t n = 1 + next_rand() % 24;
    for (uint64_t k = 0; k < n && at + k < meta; ++k) m[at + k] = (uint8_t)next_rand();
    exercise(m.data(), len);
  }
  // extreme values in each header field
  if (len >= 64) {
    const uint64_t ext[] = {0, 1, 15, 16, 64, len - 16, len, len + 16, 1ull << 32, (1ull << 63) + 8,
                            ~0ull - 15, ~0ull};
    for (uint64_t v : ext) {
      for (int f = 0; f < 6; ++f) {
        m = blob;
        switch (f) {
          case 0: put64(m.data() + 8, v); break;                    // N
          case 1: put32(m.data() + 16, (uint32_t)v); break;         // C
          case 2: put32(m.data() + 20, (uint32_t)v); break;         // K
          case 3: put64(m.data() + 32, v); break;                   // blob_nbytes
          case 4: put64(m.data() + 40, v); break;                   // payload_base
          case 5: put16(m.data() + 4, (uint16_t)v); m[27] = (uint8_t)v; break;  // version, flags
        }
        exercise(m.data(), len);
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a) {
    FILE* f = fopen(argv[a], "rb");
    if (!f) {
      fprintf(stderr, "cannot open %s\n", argv[a]);
      return 2;
    }
    std::vector<uint8_t> blob;
    uint8_t buf[65536];
    size_t n;
    while ((n = fread(buf, 1, sizeof(buf), f)) > 0) blob.insert(blob.end(), buf, buf + n);
    fclose(f);
    fuzz_blob(blob);
  }
  printf("fuzzed %ld buffers, %ld accepted headers, %ld copy ranges%s\n", g_runs, g_ok_headers, g_ranges,
         g_fail ? ", FAILED" : "");
  return g_fail;
}
