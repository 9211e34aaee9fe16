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

// Unsigned dynamic 8-bit encoder (n >= 0): buckets over the bit pattern of n,
// 7 mantissa bits per bucket (the unsigned code is twice as dense as the
// signed one); every n below 2^-22 shares bucket 0, which holds the smallest
// decision threshold (1.625e-7) and ends below the next (5.5e-7).  Starting
// there rather than a binade lower keeps the two-state optimizer kernel's LDS
// at 7 workgroups per CU.
constexpr uint32_t kUDynLowBits = 105u << 23;   // 2^-22
constexpr int kUDynShift = 16;
constexpr int kUDynBase = int(kUDynLowBits >> kUDynShift);
constexpr int kUDynLutN = int(kOneBits >> kUDynShift) - kUDynBase + 1;   // 2817
constexpr int kUDynBucketBytes = (kUDynLutN + 3) / 4 * 4;                 // 2820

// 4-bit encoders: linear buckets of n in [-1, 1]: b = (int)(n*16 + 16).
constexpr int k4LutN = 33;

// Encoder of a user code: linear buckets of n clamped to [-1, 1],
// b = (int)(n*2048 + 2048) in [0, 4096] (n*2048 is exact, so the sum rounds
// once, fused or not; a NaN n takes bucket 0).  The map is monotone, so a
// threshold in an earlier bucket is below n and one in a later bucket above
// it: with first[b] = #{k < 255 : bucket(thr[k]) < b}, b = 0..4097, the code
// of n is first[b] plus the count of bucket b's thresholds thr[first[b] ..
// first[b+1]) that are <= n.  One function for the host table and the device
// encoder (constexpr, so device code may call it).
constexpr int kUserBuckets = 4097;
constexpr int kUserFirstBytes = 4112;           // first[0 .. 4097], zero padded
constexpr int user_bucket(float n)
{
    return (int)(__builtin_fminf(__builtin_fmaxf(n, -1.0f), 1.0f) * 2048.0f + 2048.0f);
}

struct LutEntry {
    uint32_t t;        // decision threshold (binary32 bits)
    uint32_t payload;  // DYN8: 127 + thresholds below the bucket; NF4: code below (above: + 1);
                       // FP4: code below | code above << 8
};

// Dynamic 8-bit encoder.  The code is monotone in n, so with the 255 signed
// decision thresholds T[c] (smallest binary32 that encodes to c+1 or above;
// T[255] = +inf) the code of n is c + (n >= T[c]) once c, the code at the
// start of n's bucket, is known.  Buckets split |n| by its bit pattern (6
// mantissa bits each), separately for each sign; no bucket holds two
// thresholds.  dyn8_base[s][b] is c for sign s (0: n >= 0, 1: n < 0) and
// bucket b; dyn8_thr[c] holds T[c] as binary32 bits.
constexpr int kDynBucketBytes = (kDynLutN + 3) / 4 * 4;   // 1412

struct QbTables {
    float dyn8[256];               // decode, by stored code
    float nf4[16];
    float fp4[16];
    uint8_t dyn8_base[2][kDynBucketBytes];
    uint32_t dyn8_thr[256];
    LutEntry nf4_lut[k4LutN];
    LutEntry fp4_lut[k4LutN];
    // unsigned dynamic code: decode, and the encoder of n >= 0 (udyn8_base[b]
    // is the code at the start of bucket b, udyn8_thr[c] the threshold T[c])
    float udyn8[256];
    uint8_t udyn8_base[kUDynBucketBytes];
    uint32_t udyn8_thr[256];
};

// Builds every table; returns 0, or a negative value if a self-check fails.
int build_tables(QbTables* t);

// The tables, built on first use (thread-safe); nullptr if the build failed.
const QbTables* host_tables();

// The linear 8-bit code k/127, k = -128..127 (each entry rounded once).
void linear_code(float* out /* [256] */);

// Decision thresholds of a user code: values[256] must be finite and
// non-decreasing; thr[k] = smallest binary32 encoding to entry k+1 or above
// (the midpoint of the entries computed in binary64; a tie goes to the entry
// of smaller magnitude, between equal magnitudes to the upper one),
// thr[255] = +inf.  Returns 0, or -1 for an invalid code.
int user_code_thresholds(const float* values, float* thr);

// The bucket index of a user code's thresholds (the map above): first[b] for
// b = 0..4097 from thr[0..254] (ascending), zeros up to kUserFirstBytes.
void user_code_first(const float* thr, uint8_t* first /* [kUserFirstBytes] */);

}  // namespace qb
