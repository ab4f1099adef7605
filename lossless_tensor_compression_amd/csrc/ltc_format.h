// ltc_format.h -- fixed sizes of the blob format (include/ltc.h), shared by
// the device code and the host-only parsing in ltc_host.cpp.  Plain C++, no
// HIP, so the host parsing also builds with an ordinary compiler (and its
// sanitizers).
#pragma once

#include <stdint.h>

namespace ltc {

constexpr uint32_t kTotal = 4096;       // normalised frequency total (2^12)
constexpr uint32_t kLanes = 64;         // interleaved rANS lanes = one wave64
constexpr uint32_t kRansLow = 65536;    // state lower bound 2^16
constexpr uint32_t kHeader = 64;
constexpr uint32_t kDirEntry = 16;
constexpr uint32_t kRansFixed = 272;    // 16-byte prefix + 64 u32 states
constexpr uint32_t kProbBits = 12;

}  // namespace ltc
