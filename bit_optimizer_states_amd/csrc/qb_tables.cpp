// qb_tables.cpp -- host construction of the codes, their decision thresholds
// and the bucketed encoder tables.
//
// Codes (readings of the pages; the tables are not printed there):
//  * dynamic 8-bit code (abstract quoted on "Py之bitsandbytes", section 2:
//    dynamic quantization, precise for large and small magnitudes): for
//    decades e = 0..6, the 2^e midpoints of equal bins of [0.1, 1] scaled by
//    10^(e-6), i.e. (2^(e+1) + 18j + 9) / (2^(e+1) 10^(7-e)), their negatives,
//    0 and +1, sorted (256 entries);
//  * unsigned dynamic 8-bit code, for a state that is never negative (same
//    abstract; the pages name only the signed code): the sign bit becomes one
//    more fraction bit, so decade e holds the 2^(e+1) midpoints of equal bins
//    of [0.1, 1] scaled by 10^(e-6), i.e. (2^(e+2) + 18j + 9) /
//    (2^(e+2) 10^(7-e)), plus 0 and +1 (256 entries);
//  * NF4 ("Bitsandbytes", section Normal Float 4 (NF4)): quantiles of N(0,1)
//    at 1/2 + (P-1/2)k/8 (k = 1..8) and their mirrored counterparts at k/7
//    (k = 1..7), plus 0, over the quantile at P = 1 - (1/30 + 1/32)/2;
//  * FP4 ("Quantize 🤗 Transformers models", section FP4 quantization): E2M1
//    magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} / 6, sign-magnitude nibble.
//
// Encoding is nearest-entry with ties toward the entry of smaller magnitude.
// Instead of comparing against midpoints at run time, the decision threshold
// between two adjacent entries is precomputed as the smallest binary32 value
// that encodes to the upper entry; counting thresholds <= n then gives the
// code exactly, for every binary32 n.
#include "qb_tables.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

namespace qb {
namespace {

uint32_t bits_of(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float float_of(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// Nearest-even binary32 of the positive rational num/den (num, den < 2^44),
// by integer long division; results lie in the normal range here.
float rn32_ratio(uint64_t num, uint64_t den)
{
    if (num == 0) return 0.0f;
    int s = 0;  // q = floor(num * 2^s / den) must land in [2^23, 2^24)
    auto q_of = [&](int sh, unsigned __int128* rem) {
        unsigned __int128 a = sh >= 0 ? ((unsigned __int128)num << sh) : (unsigned __int128)(num >> -sh);
        unsigned __int128 q = a / den;
        if (rem) *rem = a % den;
        return q;
    };
    while (q_of(s, nullptr) >= ((unsigned __int128)1 << 24)) --s;
    while (q_of(s, nullptr) < ((unsigned __int128)1 << 23)) ++s;
    unsigned __int128 r;
    uint64_t q = (uint64_t)q_of(s, &r);
    unsigned __int128 twice = r * 2;
    if (twice > den || (twice == den && (q & 1))) ++q;
    return std::ldexp((float)q, -s);   // q <= 2^24: exact
}

void build_dyn8(float* out)
{
    std::vector<float> pos;
    for (int e = 0; e <= 6; ++e) {
        uint64_t p10 = 1;
        for (int k = 0; k < 7 - e; ++k) p10 *= 10;
        for (int j = 0; j < (1 << e); ++j)
            pos.push_back(rn32_ratio((2ull << e) + 18ull * j + 9ull, (2ull << e) * p10));
    }
    std::sort(pos.begin(), pos.end());
    for (int i = 0; i < 127; ++i) out[i] = -pos[126 - i];
    out[127] = 0.0f;
    for (int i = 0; i < 127; ++i) out[128 + i] = pos[i];
    out[255] = 1.0f;
}

void build_udyn8(float* out)
{
    std::vector<float> pos;
    for (int e = 0; e <= 6; ++e) {
        uint64_t p10 = 1;
        for (int k = 0; k < 7 - e; ++k) p10 *= 10;
        for (int j = 0; j < (2 << e); ++j)
            pos.push_back(rn32_ratio((4ull << e) + 18ull * j + 9ull, (4ull << e) * p10));
    }
    std::sort(pos.begin(), pos.end());
    out[0] = 0.0f;
    for (int i = 0; i < 254; ++i) out[1 + i] = pos[i];
    out[255] = 1.0f;
}

// Standard normal quantile by Newton's method on the CDF 1/2 erfc(-x/sqrt 2).
long double normal_quantile(long double p)
{
    const long double rs2 = 0.70710678118654752440084436210484903928L;
    const long double rs2pi = 0.39894228040143267793994605993438186848L;
    long double x = 0.0L;
    for (int it = 0; it < 200; ++it) {
        long double cdf = 0.5L * std::erfc(-x * rs2);
        long double pdf = rs2pi * std::exp(-0.5L * x * x);
        long double dx = (cdf - p) / pdf;
        x -= dx;
        if (std::fabs(dx) <= 1e-19L * (1.0L + std::fabs(x))) break;
    }
    return x;
}

void build_nf4(float* out)
{
    const long double P = 1.0L - (1.0L / 30.0L + 1.0L / 32.0L) / 2.0L;
    const long double top = normal_quantile(P);
    int n = 0;
    for (int k = 7; k >= 1; --k)
        out[n++] = (k == 7) ? -1.0f : (float)(-normal_quantile(0.5L + (P - 0.5L) * k / 7.0L) / top);
    out[n++] = 0.0f;
    for (int k = 1; k <= 8; ++k)
        out[n++] = (k == 8) ? 1.0f : (float)(normal_quantile(0.5L + (P - 0.5L) * k / 8.0L) / top);
}

void build_fp4(float* out)
{
    // E2M1 magnitude / 6 as exact ratios, by bit pattern k
    static const uint64_t num[8] = {0, 1, 1, 1, 1, 1, 2, 1};
    static const uint64_t den[8] = {1, 12, 6, 4, 3, 2, 3, 1};
    for (int k = 0; k < 8; ++k) {
        float m = rn32_ratio(num[k], den[k]);
        out[k] = m;
        out[8 + k] = k ? -m : 0.0f;
    }
}

// Smallest binary32 >= d (inclusive) or > d (strict).
float ceil_f32(double d, bool strict)
{
    float f = (float)d;
    if ((double)f < d || (strict && (double)f == d)) f = std::nextafter(f, INFINITY);
    return f;
}

// Decision thresholds of an ascending list: t[i] = smallest binary32 that
// encodes to vals[i+1] rather than vals[i].
std::vector<float> thresholds(const std::vector<float>& vals)
{
    std::vector<float> t;
    for (size_t i = 0; i + 1 < vals.size(); ++i) {
        double mid = ((double)vals[i] + (double)vals[i + 1]) / 2.0;   // exact
        bool tie_to_lower = std::fabs(vals[i]) < std::fabs(vals[i + 1]);
        t.push_back(ceil_f32(mid, tie_to_lower));
    }
    return t;
}

int build_dyn8_lut(const float* dyn8, uint8_t (*base)[kDynBucketBytes], uint32_t* thr)
{
    std::vector<float> vals(dyn8, dyn8 + 256);
    std::vector<float> T = thresholds(vals);            // 255 signed thresholds, ascending
    for (int c = 0; c < 256; ++c) thr[c] = c < 255 ? bits_of(T[c]) : 0x7F800000u;
    for (int sign = 0; sign < 2; ++sign) {
        for (int b = 0; b < kDynLutN; ++b) {
            // magnitudes of bucket b: [mlo, mhi] (bucket 0 also takes every |n| below 2^-22,
            // the last bucket only 1.0)
            const float mlo = b == 0 ? 0.0f : float_of(uint32_t(b + kDynBase) << kDynShift);
            const float mhi = b == kDynLutN - 1 ? 1.0f : float_of((uint32_t(b + kDynBase + 1) << kDynShift) - 1u);
            const float lo = sign ? -mhi : mlo, hi = sign ? -mlo : mhi;   // n in [lo, hi]
            int c = 0;
            while (c < 255 && T[c] <= lo) ++c;            // code at n = lo
            if (c + 1 < 255 && T[c + 1] <= hi) return -1;  // two thresholds in one bucket
            base[sign][b] = (uint8_t)c;
        }
    }
    return 0;
}

int build_udyn8_lut(const float* udyn8, uint8_t* base, uint32_t* thr)
{
    std::vector<float> vals(udyn8, udyn8 + 256);
    std::vector<float> T = thresholds(vals);            // 255 thresholds, ascending
    for (int c = 0; c < 256; ++c) thr[c] = c < 255 ? bits_of(T[c]) : 0x7F800000u;
    for (int b = 0; b < kUDynLutN; ++b) {
        // n of bucket b: [lo, hi] (bucket 0 also takes every n below 2^-22, the last only 1.0)
        const float lo = b == 0 ? 0.0f : float_of(uint32_t(b + kUDynBase) << kUDynShift);
        const float hi = b == kUDynLutN - 1 ? 1.0f : float_of((uint32_t(b + kUDynBase + 1) << kUDynShift) - 1u);
        int c = 0;
        while (c < 255 && T[c] <= lo) ++c;
        if (c + 1 < 255 && T[c + 1] <= hi) return -1;  // two thresholds in one bucket
        base[b] = (uint8_t)c;
    }
    return 0;
}

// The device takes the bucket of n in [-1, 1] as 16 n + 16 rounded once to
// the nearest integer, ties to even (one fused multiply-add onto 1.5 * 2^23,
// whose float bits then hold the bucket).  In binary64 16 n is exact and the
// sum can round only far from a tie (near k + 1/2, 16 n has an ulp of at
// least 2^-25), so nearbyint of the binary64 sum is the same bucket.
int bucket4(float n)
{
    const double u = (double)n * 16.0 + 16.0;
    const int b = (int)std::nearbyint(u);
    return b < 0 ? 0 : (b > k4LutN - 1 ? k4LutN - 1 : b);
}

uint32_t order_key(float f)
{
    uint32_t u = bits_of(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

float from_key(uint32_t k)
{
    return float_of((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Smallest binary32 n in [-1, 1] with bucket4(n) >= b (bisection on the order).
float bucket_start(int b)
{
    uint32_t lo = order_key(-1.0f), hi = order_key(1.0f);
    if (bucket4(-1.0f) >= b) return -1.0f;
    while (hi - lo > 1) {
        uint32_t mid = lo + (hi - lo) / 2;
        if (bucket4(from_key(mid)) >= b) hi = mid; else lo = mid;
    }
    return from_key(hi);
}

// vals: distinct values ascending; codes: the stored code of each value.
// sorted: the codes ascend with the values (NF4), so the code above a
// threshold is always the one below plus 1 and the payload holds only the
// code below; otherwise (FP4) it holds both.
int build_4bit_lut(const std::vector<float>& vals, const std::vector<uint32_t>& codes, bool sorted, LutEntry* lut)
{
    std::vector<float> t = thresholds(vals);
    const int nt = (int)t.size();
    for (int b = 0; b < k4LutN; ++b) {
        float lo = bucket_start(b);
        float hi = b + 1 < k4LutN ? std::nextafter(bucket_start(b + 1), -INFINITY) : 1.0f;
        int k = 0;
        while (k < nt && t[k] <= lo) ++k;
        if (k + 1 < nt && t[k + 1] <= hi) return -1;
        lut[b].t = k < nt ? bits_of(t[k]) : 0x7F800000u;
        uint32_t below = codes[k], above = codes[k < nt ? k + 1 : k];
        if (sorted && k < nt && t[k] <= hi && above != below + 1) return -1;
        lut[b].payload = sorted ? below : (below | (above << 8));
    }
    return 0;
}

// Direct nearest search (ties toward zero), used only to self-check the tables.
int nearest(const std::vector<float>& vals, float x)
{
    int best = 0;
    for (int i = 1; i < (int)vals.size(); ++i) {
        double db = std::fabs((double)x - vals[best]), di = std::fabs((double)x - vals[i]);
        if (di < db || (di == db && std::fabs(vals[i]) < std::fabs(vals[best]))) best = i;
    }
    return best;
}

int self_check(const QbTables* T)
{
    // a deterministic sweep of [-1, 1]: the bucket encoders against the direct search
    std::vector<float> dyn(T->dyn8, T->dyn8 + 256);
    std::vector<float> nf4(T->nf4, T->nf4 + 16);
    std::vector<float> udyn(T->udyn8, T->udyn8 + 256);
    uint32_t state = 12345u;
    for (int i = 0; i < 200000; ++i) {
        state = state * 1664525u + 1013904223u;
        float x = (i & 1) ? std::ldexp((float)(state >> 8) / 16777216.0f, -(int)(i % 30))
                          : (float)(state >> 8) / 8388608.0f - 1.0f;
        if (i & 2) x = -x;
        if (!(x >= -1.0f && x <= 1.0f)) continue;
        uint32_t mag = bits_of(x) & 0x7FFFFFFFu;
        uint32_t cl = std::min(std::max(mag, kDynLowBits), kOneBits);
        const int c0 = T->dyn8_base[bits_of(x) >> 31][(cl >> kDynShift) - kDynBase];
        int code = c0 + (x >= float_of(T->dyn8_thr[c0]) ? 1 : 0);
        if (code != nearest(dyn, x)) return -10;
        const LutEntry& f = T->nf4_lut[bucket4(x)];
        const int c4 = (int)f.payload + (x >= float_of(f.t) ? 1 : 0);
        if (c4 != nearest(nf4, x)) return -11;
        // the unsigned encoder on |x|
        const float ax = std::fabs(x);
        const uint32_t ucl = std::min(std::max(bits_of(ax), kUDynLowBits), kOneBits);
        const int u0 = T->udyn8_base[(ucl >> kUDynShift) - kUDynBase];
        if (u0 + (ax >= float_of(T->udyn8_thr[u0]) ? 1 : 0) != nearest(udyn, ax)) return -12;
    }
    return 0;
}

}  // namespace

int build_tables(QbTables* T)
{
    std::memset(T, 0, sizeof(*T));
    build_dyn8(T->dyn8);
    build_nf4(T->nf4);
    build_fp4(T->fp4);
    for (int i = 0; i < 255; ++i)
        if (!(T->dyn8[i] < T->dyn8[i + 1])) return -2;
    if (build_dyn8_lut(T->dyn8, T->dyn8_base, T->dyn8_thr) != 0) return -3;
    build_udyn8(T->udyn8);
    for (int i = 0; i < 255; ++i)
        if (!(T->udyn8[i] < T->udyn8[i + 1])) return -6;
    if (build_udyn8_lut(T->udyn8, T->udyn8_base, T->udyn8_thr) != 0) return -7;

    std::vector<float> nf4(T->nf4, T->nf4 + 16);
    std::vector<uint32_t> nf4_codes(16);
    for (int i = 0; i < 16; ++i) nf4_codes[i] = (uint32_t)i;
    if (build_4bit_lut(nf4, nf4_codes, true, T->nf4_lut) != 0) return -4;

    // FP4 as a line of 15 distinct values: -mag[7..1], 0, mag[1..7]
    std::vector<float> fp4;
    std::vector<uint32_t> fp4_codes;
    for (int k = 7; k >= 1; --k) { fp4.push_back(T->fp4[8 + k]); fp4_codes.push_back(8u | (uint32_t)k); }
    fp4.push_back(0.0f); fp4_codes.push_back(0u);
    for (int k = 1; k <= 7; ++k) { fp4.push_back(T->fp4[k]); fp4_codes.push_back((uint32_t)k); }
    if (build_4bit_lut(fp4, fp4_codes, false, T->fp4_lut) != 0) return -5;
    return self_check(T);
}

void linear_code(float* out)
{
    for (int k = -128; k <= 127; ++k) {
        const float m = rn32_ratio((uint64_t)(k < 0 ? -k : k), 127);
        out[k + 128] = k < 0 ? -m : m;
    }
}

int user_code_thresholds(const float* values, float* thr)
{
    for (int k = 0; k < 256; ++k)
        if (!std::isfinite(values[k]) || (k > 0 && !(values[k - 1] <= values[k]))) return -1;
    std::vector<float> t = thresholds(std::vector<float>(values, values + 256));
    for (int k = 0; k < 255; ++k) thr[k] = t[k];
    thr[255] = INFINITY;
    return 0;
}

void user_code_first(const float* thr, uint8_t* first)
{
    int k = 0;
    for (int b = 0; b <= kUserBuckets; ++b) {
        while (k < 255 && user_bucket(thr[k]) < b) ++k;
        first[b] = (uint8_t)k;
    }
    for (int b = kUserBuckets + 1; b < kUserFirstBytes; ++b) first[b] = 0;
}

const QbTables* host_tables()
{
    static QbTables tables;
    static int status = 1;
    static std::once_flag once;
    std::call_once(once, [] { status = build_tables(&tables); });
    return status == 0 ? &tables : nullptr;
}

}  // namespace qb
