// ltc_crc.h -- CRC-32 (zlib's: reflected polynomial 0xEDB88320, register
// preset to all ones, result complemented) building blocks shared by the
// per-chunk CRC kernel and the pack kernel that checksums the blob while it
// writes it.
//
// CRC is linear over GF(2).  With crc_raw(M) the remainder of a register that
// starts at zero,
//   crc_raw(A || B) = crc_raw(A) * x^(8|B|) mod P  xor  crc_raw(B),
// and leading zero bytes leave crc_raw unchanged.  zlib's register is preset
// to 0xFFFFFFFF at the first byte (which adds 0xFFFFFFFF * x^(8L) mod P for a
// message of L bytes), and the result is complemented.  Multiplication by a constant power of x is itself a linear
// map of the 32-bit remainder, tabulated per operand byte (four 256-entry
// tables); remainders of 16-byte units come from slicing-by-8 tables
// (Kounavis & Berry, "A Systematic Approach to Building High Performance
// Software-based CRC Generators", 2005).
#pragma once

#include "ltc_internal.h"

namespace ltc {

constexpr uint32_t kPoly = 0xEDB88320u;  // reflected CRC-32 polynomial
constexpr int kCrcLevels = 6;            // tree levels over the 64 lanes of a wave

// LDS tables: t8[m][b] (8 x 256) and, per multiplication constant l,
// tl[l][p][b] (4 x 256).  Constants 0..5 are the tree levels; a seventh can
// serve other shifts.
template <int L> struct CrcLdsT {
  static constexpr int kLevels = L;
  uint32_t t8[8][256];
  uint32_t tl[L][4][256];
  uint32_t basis[L][32];
};

// a * b mod P with bit 31 - d of a word holding the coefficient of x^d
__device__ __forceinline__ uint32_t gf2_mulmod(uint32_t a, uint32_t b) {
  uint32_t r = 0;
  for (int i = 0; i < 32; ++i) {
    if (a & (0x80000000u >> i)) r ^= b;
    b = (b >> 1) ^ (kPoly & (0u - (b & 1u)));
  }
  return r;
}

// Fills the tables; lvl[l] is multiplication constant l.  Every thread of
// the workgroup calls it; it ends with a workgroup barrier.
template <int L>
__device__ __forceinline__ void crc_build_tables(CrcLdsT<L>& s, const uint32_t* lvl, uint32_t tid,
                                                 uint32_t nthreads) {
  for (uint32_t b = tid; b < 256; b += nthreads) {
    // t8[m][b] = register after byte b followed by m zero bytes
    uint32_t c = b;
    for (int m = 0; m < 8; ++m) {
      for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (kPoly & (0u - (c & 1u)));
      s.t8[m][b] = c;
    }
  }
  // images of the 32 single-bit words under each level's multiplication
  for (uint32_t i = tid; i < L * 32; i += nthreads)
    s.basis[i / 32][i % 32] = gf2_mulmod(1u << (i % 32), lvl[i / 32]);
  __syncthreads();
  for (uint32_t idx = tid; idx < L * 4 * 256; idx += nthreads) {
    const uint32_t l = idx / 1024, p = (idx / 256) & 3, b = idx & 255;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b & (1u << i)) v ^= s.basis[l][8 * p + i];
    s.tl[l][p][b] = v;
  }
  __syncthreads();
}

// register c advanced over the 16 bytes of q (little-endian words)
template <int L>
__device__ __forceinline__ uint32_t crc_step16(const CrcLdsT<L>& s, uint32_t c, const uint4 q) {
  c ^= q.x;
  c = s.t8[7][c & 0xFFu] ^ s.t8[6][(c >> 8) & 0xFFu] ^ s.t8[5][(c >> 16) & 0xFFu] ^
      s.t8[4][c >> 24] ^ s.t8[3][q.y & 0xFFu] ^ s.t8[2][(q.y >> 8) & 0xFFu] ^
      s.t8[1][(q.y >> 16) & 0xFFu] ^ s.t8[0][q.y >> 24];
  c ^= q.z;
  c = s.t8[7][c & 0xFFu] ^ s.t8[6][(c >> 8) & 0xFFu] ^ s.t8[5][(c >> 16) & 0xFFu] ^
      s.t8[4][c >> 24] ^ s.t8[3][q.w & 0xFFu] ^ s.t8[2][(q.w >> 8) & 0xFFu] ^
      s.t8[1][(q.w >> 16) & 0xFFu] ^ s.t8[0][q.w >> 24];
  return c;
}

// c * lvl[l] mod P
template <int L>
__device__ __forceinline__ uint32_t crc_mul_level(const CrcLdsT<L>& s, int l, uint32_t c) {
  return s.tl[l][0][c & 0xFFu] ^ s.tl[l][1][(c >> 8) & 0xFFu] ^ s.tl[l][2][(c >> 16) & 0xFFu] ^
         s.tl[l][3][c >> 24];
}

// ---- bank-interleaved tables (k_crc32)
// A lookup indexed by data is a random LDS access: 64 lanes reading one
// 1 KiB table collide on most banks (the k_crc32 of a 1.2 GB blob with
// slicing-by-16 tables of this kind spent about half its time stalled on bank
// conflicts).  Here every slicing-by-4 table (table m, entry b: the register
// after byte b and m zero bytes) is stored as 32 copies interleaved by bank,
// and lane l reads copy l % 32, so the 32 lanes an LDS cycle serves hit 32
// different banks.  Copy j of entry b of table m sits at byte address
//   (m >> 1) << 16 | b << 8 | (m & 1) << 7 | j << 2,
// so a lookup's address is one byte permute: the data byte goes to address
// byte 1, the lane's (m >> 1) << 16 | j << 2 supplies bytes 0 and 2, and
// (m & 1) << 7 is the load's immediate offset.  The four tables fill 128 KiB,
// so a workgroup that holds them has a CU to itself.
struct CrcBankLds {
  uint32_t bank[4 * 256 * 32];
  uint32_t tl[kCrcLevels][4][256];
  uint32_t basis[kCrcLevels][32];
};

__host__ __device__ constexpr uint32_t crc_bank_index(uint32_t m, uint32_t b, uint32_t j) {
  return (m >> 1) << 14 | b << 6 | (m & 1) << 5 | j;
}

// Fills the tables (tl and basis as crc_build_tables); every thread of the
// workgroup calls it; it ends with a workgroup barrier.
__device__ __forceinline__ void crc_build_bank(CrcBankLds& s, const uint32_t* lvl, uint32_t tid,
                                               uint32_t nthreads) {
  for (uint32_t b = tid; b < 256; b += nthreads) {  // copy 0
    uint32_t c = b;
    for (int m = 0; m < 4; ++m) {
      for (int k = 0; k < 8; ++k) c = (c >> 1) ^ (kPoly & (0u - (c & 1u)));
      s.bank[crc_bank_index(m, b, 0)] = c;
    }
  }
  for (uint32_t i = tid; i < kCrcLevels * 32; i += nthreads)
    s.basis[i / 32][i % 32] = gf2_mulmod(1u << (i % 32), lvl[i / 32]);
  __syncthreads();
  for (uint32_t idx = tid; idx < 4 * 256 * 32; idx += nthreads) {  // copies 1..31
    const uint32_t j = idx & 31;
    if (j) s.bank[idx] = s.bank[idx - j];
  }
  for (uint32_t idx = tid; idx < kCrcLevels * 4 * 256; idx += nthreads) {
    const uint32_t l = idx / 1024, p = (idx / 256) & 3, b = idx & 255;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (b & (1u << i)) v ^= s.basis[l][8 * p + i];
    s.tl[l][p][b] = v;
  }
  __syncthreads();
}

// entry of table m (immediate (m & 1) << 7) at address a (one byte permute)
__device__ __forceinline__ uint32_t crc_bank_at(const CrcBankLds& s, uint32_t a, uint32_t half) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(s.bank) + a + (half << 7));
}

// register c advanced over the 4 bytes of little-endian word w; bl: the
// lane's table copy (lane % 32).  v_perm_b32 selector bytes 0-3 pick bytes
// of the second operand, 4-7 of the first.
__device__ __forceinline__ uint32_t crc_word_bank(const CrcBankLds& s, uint32_t c, uint32_t w, uint32_t bl) {
  const uint32_t lb0 = bl << 2, lb1 = lb0 | 0x10000u;  // tables 0-1, tables 2-3
  c ^= w;
  return crc_bank_at(s, __builtin_amdgcn_perm(c, lb1, 0x03020400u), 1) ^  // byte 0: table 3
         crc_bank_at(s, __builtin_amdgcn_perm(c, lb1, 0x03020500u), 0) ^  // byte 1: table 2
         crc_bank_at(s, __builtin_amdgcn_perm(c, lb0, 0x03020600u), 1) ^  // byte 2: table 1
         crc_bank_at(s, __builtin_amdgcn_perm(c, lb0, 0x03020700u), 0);   // byte 3: table 0
}

__device__ __forceinline__ uint32_t crc_step16_bank(const CrcBankLds& s, uint32_t c, const uint4 q,
                                                    uint32_t bl) {
  c = crc_word_bank(s, c, q.x, bl);
  c = crc_word_bank(s, c, q.y, bl);
  c = crc_word_bank(s, c, q.z, bl);
  return crc_word_bank(s, c, q.w, bl);
}

__device__ __forceinline__ uint32_t crc_step1_bank(const CrcBankLds& s, uint32_t c, uint32_t byte,
                                                   uint32_t bl) {
  return crc_bank_at(s, __builtin_amdgcn_perm(c ^ byte, bl << 2, 0x03020400u), 0) ^ (c >> 8);
}

// Lane i holds the remainder of segment i of 64 equal consecutive segments
// (level l's constant shifts by 2^l segments).  Returns, in lane 0, the
// remainder of the concatenation; every lane of the wave must call it.
__device__ __forceinline__ uint32_t crc_tree64_bank(const CrcBankLds& s, uint32_t c, uint32_t lane) {
#pragma unroll
  for (int l = 0; l < kCrcLevels; ++l) {
    const uint32_t right = __shfl_down(c, 1u << l, 64);
    if ((lane & ((2u << l) - 1u)) == 0)
      c = (s.tl[l][0][c & 0xFFu] ^ s.tl[l][1][(c >> 8) & 0xFFu] ^ s.tl[l][2][(c >> 16) & 0xFFu] ^
           s.tl[l][3][c >> 24]) ^ right;
  }
  return c;
}

}  // namespace ltc
