// qb_tables.h -- constant tables of the codes and of their encoders.
//
// Built once on the host (qb_tables.cpp), uploaded once per device, and staged
// from there into LDS by every workgroup that needs them.
#pragma once
#include <stdint.h>

namespace qb {

// Dynamic 8-bit encoder: buckets over the binary32 bit pattern of |n|,
// 6 mantissa bits per bucket; every |n| below 2^-22 shares bucket 0 (the
// smallest decision threshold is 2.75e-7 > 2^-22).  Every bucket holds at most
// one decision threshold, so one compare finishes the search.
constexpr uint32_t kDynLowBits = 105u << 23;    // 2^-22
constexpr uint32_t kOneBits = 0x3F800000u;      // 1.0
constexpr int kDynShift = 17;
constexpr int kDynBase = int(kDynLowBits >> kDynShift);
constexpr int kDynLutN = int(kOneBits >> kDynShift) - kDynBase + 1;   // 1409

// 4-bit encoders: linear buckets of n in [-1, 1]: b = (int)(n*16 + 16).
constexpr int k4LutN = 33;

struct LutEntry {
    uint32_t t;        // decision threshold (binary32 bits)
    uint32_t payload;  // DYN8: 127 + thresholds below the bucket; 4-bit: code below | code above << 8
};

struct QbTables {
    float dyn8[256];               // decode, by stored code
    float nf4[16];
    float fp4[16];
    LutEntry dyn8_lut[kDynLutN];
    LutEntry nf4_lut[k4LutN];
    LutEntry fp4_lut[k4LutN];
    float pair[2][256][2];         // [nf4, fp4][byte] -> {value of high nibble, value of low nibble}
};

// Builds every table; returns 0, or a negative value if a self-check fails.
int build_tables(QbTables* t);

// The tables, built on first use (thread-safe); nullptr if the build failed.
const QbTables* host_tables();

}  // namespace qb
