// qb_codes.hip -- estimation of a quantile code from data.
//
// The pages list quantile quantization among the 8-bit types and a fast
// quantile estimation ("Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细
// 攻略", section 1).  The code entries are the midpoints of adjacent quantiles
// of the data at probabilities j/257, j = 0..256, normalized to a largest
// magnitude of 1.  The quantiles are estimated fast and deterministically:
//   1. k_chunk_quantiles: one workgroup per chunk of 4096 consecutive values
//      sorts the chunk (bitonic network: 16 values per thread in registers,
//      lane shuffles within a wave, LDS only across waves) and keeps its 257 order
//      statistics s[floor(j L / 257)] (L = the chunk's length);
//   2. k_quantile_means: one workgroup per statistic j adds its chunks'
//      values exactly (integer sums of the significands per binary exponent)
//      and divides once: A_j = the exact mean, rounded to nearest-even
//      binary64, whatever the order of the additions;
//   3. k_quantile_code forms the midpoints, normalizes them and writes the
//      code with its decision thresholds and their bucket index.
// Every step is exact or a fixed sequence of IEEE operations, so the result is
// the same bits on every run.
#include "qb_device.h"

namespace qb {

namespace {

constexpr int kSortPerThread = kQuantileChunk / kThreads;   // 16 consecutive elements per thread
constexpr int kExpBins = 254;                                // binary32 exponents 1..254 (0 joins 1)
constexpr int kWaveElems = 64 * kSortPerThread;              // 1024 elements per wave
constexpr int kWaveShift = 10;

// LDS slot of chunk element i: one pad word per 32 keeps the lane-strided
// accesses (lane stride 16 words) at two-way bank conflicts.
__device__ __forceinline__ int slot(int i) { return i + (i >> 5); }

// Compare-exchange, ascending: x takes the smaller value.
__device__ __forceinline__ void cas(float& x, float& y)
{
    const float lo = fminf(x, y), hi = fmaxf(x, y);
    x = lo;
    y = hi;
}

// Value of lane ^ M within the wave: by a DPP move for ^1, ^2, ^3 (quad
// permutations), ^7 and ^15 (the half-row and row mirrors); by the LDS
// crossbar otherwise, a swizzle within 32 lanes for ^4, ^8, ^16 (no address
// operand) and a permute for ^31, ^32, ^63.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int M>
__device__ __forceinline__ float lane_xor(float x)
{
    constexpr int kQuadSwap1 = 0xB1, kQuadSwap2 = 0x4E, kQuadRev = 0x1B, kRowMirror = 0x140, kHalfMirror = 0x141;
    if constexpr (M == 1) return dpp<kQuadSwap1>(x);
    else if constexpr (M == 2) return dpp<kQuadSwap2>(x);
    else if constexpr (M == 3) return dpp<kQuadRev>(x);
    else if constexpr (M == 7) return dpp<kHalfMirror>(x);
    else if constexpr (M == 15) return dpp<kRowMirror>(x);
    else if constexpr (M == 4 || M == 8 || M == 16)      // swizzle, bit-mask mode: lane ^ M within 32 lanes
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (M << 10) | 0x1F));
    else return __shfl_xor(x, M);
}

// A lane-shuffle stage keeps min(v, w) in the lower lane of a pair and
// max(v, w) in the upper one: med3(v, w, -inf) and med3(v, w, +inf), one
// instruction with a per-lane third operand (the values are finite or +inf).
__device__ __forceinline__ float keep_bound(bool lower) { return lower ? -INFINITY : INFINITY; }

// One lane-shuffle stage: element r of this lane meets element r (MIRROR:
// element 15 - r) of lane ^ M; the lower lane of the pair keeps the minimum.
template <int M, bool MIRROR>
__device__ __forceinline__ void lane_stage(float* v, bool lower)
{
    const float keep = keep_bound(lower);
    float w[kSortPerThread];
#pragma unroll
    for (int r = 0; r < kSortPerThread; ++r) w[r] = lane_xor<M>(v[MIRROR ? kSortPerThread - 1 - r : r]);
#pragma unroll
    for (int r = 0; r < kSortPerThread; ++r) v[r] = __builtin_amdgcn_fmed3f(v[r], w[r], keep);
}

// Bitonic sort (ascending) of the chunk, in the form without directions: the
// merge of two sorted runs of size/2 into a sorted run of `size` first pairs
// element i with its mirror i ^ (size - 1), then i with i ^ stride for
// stride = size/4 .. 1; every compare-exchange puts the smaller value at the
// lower index, so no step selects on a direction.  Thread t holds elements
// 16 t .. 16 t + 15 in registers; pairs within a thread (stride < 16) run in
// registers, pairs across lanes by lane shuffles, pairs across waves (stride
// >= 1024) through LDS.
template <int XDT>
__global__ __launch_bounds__(kThreads) void k_chunk_quantiles(const void* __restrict__ x, int64_t n, int64_t nchunks,
                                                              float* __restrict__ E)
{
    __shared__ float s[kQuantileChunk + kQuantileChunk / 32];
    const int tid = threadIdx.x;
    const int64_t c = blockIdx.x;
    const int64_t lo = c * kQuantileChunk;
    const int L = (int)(n - lo < kQuantileChunk ? n - lo : kQuantileChunk);
    const int base = tid * kSortPerThread;
    float v[kSortPerThread];
#pragma unroll
    for (int r = 0; r < kSortPerThread; ++r) {
        const int i = base + r;
        float t = INFINITY;                                    // padding sorts to the end
        if (i < L) {
            t = load1<XDT>(x, lo + i);
            t = t == 0.0f ? 0.0f : t;                          // -0 counts as +0
        }
        v[r] = t;
    }
    // sizes 2 .. 16: wholly inside a thread
#pragma unroll
    for (int size = 2; size <= kSortPerThread; size <<= 1) {
#pragma unroll
        for (int r = 0; r < kSortPerThread; ++r)
            if ((r & (size >> 1)) == 0) cas(v[r], v[r ^ (size - 1)]);
#pragma unroll
        for (int stride = size >> 2; stride > 0; stride >>= 1)
#pragma unroll
            for (int r = 0; r < kSortPerThread; ++r)
                if ((r & stride) == 0) cas(v[r], v[r + stride]);
    }
    // sizes 32 .. 4096
    for (int size = 2 * kSortPerThread; size <= kQuantileChunk; size <<= 1) {
        int top;                                               // the largest lane-shuffle stride
        if (size > kWaveElems) {
            // the mirror stage and strides >= 1024 pair elements of different
            // waves: through LDS, 8 pairs per thread
#pragma unroll
            for (int r = 0; r < kSortPerThread; ++r) s[slot(base + r)] = v[r];
            __syncthreads();
            for (int ls = __builtin_ctz(size) - 1; ls >= kWaveShift; --ls) {
                const int stride = 1 << ls;
                const bool mirror = stride == size >> 1;
#pragma unroll
                for (int k = 0; k < kSortPerThread / 2; ++k) {
                    const int q = k * kThreads + tid;          // pair q: i has a zero at bit `stride`
                    const int i = ((q >> ls) << (ls + 1)) | (q & (stride - 1));
                    const int j = mirror ? i ^ (size - 1) : i + stride;
                    float a = s[slot(i)], b = s[slot(j)];
                    cas(a, b);
                    s[slot(i)] = a;
                    s[slot(j)] = b;
                }
                __syncthreads();
            }
#pragma unroll
            for (int r = 0; r < kSortPerThread; ++r) v[r] = s[slot(base + r)];
            __syncthreads();                                   // before the next size overwrites s
            top = kWaveElems >> 1;
        } else {
            // the mirror stage within the wave: element 16 t + r pairs with
            // element 15 - r of lane t ^ (size/16 - 1)
            const bool lower = (tid & (size / (2 * kSortPerThread))) == 0;
            switch (size / kSortPerThread - 1) {           // wave-uniform
            case 1: lane_stage<1, true>(v, lower); break;
            case 3: lane_stage<3, true>(v, lower); break;
            case 7: lane_stage<7, true>(v, lower); break;
            case 15: lane_stage<15, true>(v, lower); break;
            case 31: lane_stage<31, true>(v, lower); break;
            default: lane_stage<63, true>(v, lower); break;
            }
            top = size >> 2;
        }
        for (int stride = top; stride >= kSortPerThread; stride >>= 1) {
            const int lanes = stride / kSortPerThread;
            const bool lower = (tid & lanes) == 0;
            switch (lanes) {                                   // wave-uniform
            case 1: lane_stage<1, false>(v, lower); break;
            case 2: lane_stage<2, false>(v, lower); break;
            case 4: lane_stage<4, false>(v, lower); break;
            case 8: lane_stage<8, false>(v, lower); break;
            case 16: lane_stage<16, false>(v, lower); break;
            default: lane_stage<32, false>(v, lower); break;
            }
        }
#pragma unroll
        for (int stride = kSortPerThread >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int r = 0; r < kSortPerThread; ++r)
                if ((r & stride) == 0) cas(v[r], v[r + stride]);
    }
#pragma unroll
    for (int r = 0; r < kSortPerThread; ++r) s[slot(base + r)] = v[r];
    __syncthreads();
    for (int j = tid; j < 257; j += kThreads) E[(int64_t)j * nchunks + c] = s[slot((int)((int64_t)j * L / 257))];
}

// ---------------------------------------------------------------------------
// exact mean of each statistic over the chunks
// ---------------------------------------------------------------------------

// Bits [pos, pos + 128) of the non-negative integer w[0..5] (64-bit words,
// little-endian), pos >= 0.
__device__ unsigned __int128 bits128(const unsigned long long* w, int pos)
{
    unsigned __int128 r = 0;
    for (int k = 0; k < 2; ++k) {
        const int b = pos + 64 * k, q = b >> 6, s = b & 63;
        unsigned long long v = q < 6 ? (w[q] >> s) : 0ull;
        if (s && q + 1 < 6) v |= w[q + 1] << (64 - s);
        r |= (unsigned __int128)v << (64 * k);
    }
    return r;
}

// N 2^-149 / count rounded once to nearest-even binary64, for the integer
// N = sum_b bins[b] 2^b (signed bins) and 0 < count < 2^31.  One thread.
// |N| < 2^310 is formed exactly in 384-bit two's complement; its top 96 bits
// W (shifted up when |N| is shorter) are divided by count, which leaves a
// quotient Q of at least 64 bits; Q's top 53 bits, the next one and a sticky
// bit (Q's lower bits, the remainder, |N|'s bits below the window) round it.
__device__ double mean_rn64(const long long* bins, const unsigned long long* mask, uint32_t count)
{
    unsigned long long w[6] = {0, 0, 0, 0, 0, 0};
    for (int q = 0; q < 4; ++q) {
        unsigned long long mk = mask[q];
        while (mk) {
            const int b = q * 64 + __ffsll((long long)mk) - 1;
            mk &= mk - 1;
            const long long v = bins[b];
            const unsigned long long ext = v < 0 ? ~0ull : 0ull;   // sign extension above the value
            const int wi = b >> 6, s = b & 63;
            const unsigned long long part[3] = {(unsigned long long)v << s,
                                                s ? ((unsigned long long)v >> (64 - s)) | (ext << s) : ext, ext};
            unsigned long long carry = 0;
            for (int k = wi; k < 6; ++k) {
                const unsigned long long add = k - wi < 3 ? part[k - wi] : ext;
                const unsigned long long t = w[k] + add;
                const unsigned long long c1 = t < w[k] ? 1ull : 0ull;
                w[k] = t + carry;
                carry = c1 + (w[k] < t ? 1ull : 0ull);
            }
        }
    }
    const bool neg = (w[5] >> 63) != 0;
    if (neg) {                                                   // magnitude
        unsigned long long carry = 1;
        for (int k = 0; k < 6; ++k) {
            w[k] = ~w[k] + carry;
            carry = (carry && w[k] == 0) ? 1ull : 0ull;
        }
    }
    int top = 5;
    while (top >= 0 && w[top] == 0) --top;
    if (top < 0) return 0.0;
    const int L = top * 64 + 63 - __clzll((long long)w[top]);   // top set bit of |N|
    const int sh = L - 95;                                       // window [sh, sh + 96)
    unsigned __int128 W;
    bool low_nz = false;
    if (sh >= 0) {
        W = bits128(w, sh) & ((((unsigned __int128)1) << 96) - 1);
        for (int q = 0; q < 6 && q * 64 < sh; ++q) {
            const int nbits = sh - q * 64;
            const unsigned long long mk = nbits >= 64 ? ~0ull : ((1ull << nbits) - 1ull);
            if (w[q] & mk) low_nz = true;
        }
    } else {
        W = bits128(w, 0) << (-sh);                             // |N| < 2^95: exact
    }
    const uint32_t l2 = (uint32_t)(W >> 64), l1 = (uint32_t)(W >> 32), l0 = (uint32_t)W;
    unsigned long long cur = l2;
    const unsigned long long q2 = cur / count;
    unsigned long long r = cur % count;
    cur = (r << 32) | l1;
    const unsigned long long q1 = cur / count;
    r = cur % count;
    cur = (r << 32) | l0;
    const unsigned long long q0 = cur / count;
    r = cur % count;
    const unsigned __int128 Q = ((unsigned __int128)q2 << 64) + ((unsigned __int128)q1 << 32) + q0;
    const unsigned long long qhi = (unsigned long long)(Q >> 64), qlo = (unsigned long long)Q;
    const int H = qhi ? 64 + 63 - __clzll((long long)qhi) : 63 - __clzll((long long)qlo);   // >= 64
    const int srel = H - 52;
    const unsigned long long mant = (unsigned long long)(Q >> srel);
    const bool guard = (unsigned long long)(Q >> (srel - 1)) & 1ull;
    const unsigned __int128 below = Q & ((((unsigned __int128)1) << (srel - 1)) - 1);
    const bool up = guard && (below != 0 || r != 0 || low_nz || (mant & 1ull));
    // value = (mant + up) 2^(srel + sh - 149); the implicit bit of mant
    // carries into the exponent field
    const unsigned long long bits = ((unsigned long long)(srel + sh + 925) << 52) + mant + (up ? 1ull : 0ull);
    const double a = __longlong_as_double((long long)bits);
    return neg ? -a : a;
}

// Workgroup j: A[j] = the exact mean of E[j][0 .. nchunks), rounded once.
// Each thread adds its chunks' significands (signed) into a running sum per
// exponent, flushing to the LDS bins when the exponent changes; the bins are
// 64-bit integers, so every order of additions gives the same sums.
__global__ __launch_bounds__(kThreads) void k_quantile_means(const float* __restrict__ E, int64_t nchunks,
                                                             double* __restrict__ A)
{
    __shared__ long long s_bins[256];
    __shared__ unsigned long long s_mask[4];
    const int tid = threadIdx.x;
    s_bins[tid] = 0;
    __syncthreads();
    const float* row = E + (int64_t)blockIdx.x * nchunks;
    int cur = -1;
    long long acc = 0;
    for (int64_t c = tid; c < nchunks; c += kThreads) {
        const uint32_t u = fbits(row[c]);
        const uint32_t e = (u >> 23) & 0xFFu;
        const long long m = (long long)((u & 0x7FFFFFu) | (e ? 0x800000u : 0u));
        const int b = (int)(e ? e : 1u) - 1;
        if (b != cur) {
            if (acc) atomicAdd((unsigned long long*)&s_bins[cur], (unsigned long long)acc);
            cur = b;
            acc = 0;
        }
        acc += (u >> 31) ? -m : m;
    }
    if (acc) atomicAdd((unsigned long long*)&s_bins[cur], (unsigned long long)acc);
    __syncthreads();
    const unsigned long long mk = __ballot(tid < kExpBins && s_bins[tid] != 0);
    if ((tid & 63) == 0) s_mask[tid >> 6] = mk;
    __syncthreads();
    if (tid == 0) A[blockIdx.x] = mean_rn64(s_bins, s_mask, (uint32_t)nchunks);
}

// The next binary32 above finite f (above +-0: the smallest subnormal).
__device__ float next_up(float f)
{
    if (f == 0.0f) return ffrom(1u);
    return ffrom(f > 0.0f ? fbits(f) + 1u : fbits(f) - 1u);
}

// Smallest binary32 >= d (> d when strict), d finite.
__device__ float ceil_f32(double d, bool strict)
{
    float f = (float)d;
    if ((double)f < d || (strict && (double)f == d)) f = next_up(f);
    return f;
}

__global__ __launch_bounds__(kThreads) void k_quantile_code(const double* __restrict__ Ag,
                                                            double* __restrict__ averages, UserCode* __restrict__ out)
{
    __shared__ double A[257];
    __shared__ double q[256];
    __shared__ double red[kThreads / 64];
    __shared__ float vals[256];
    __shared__ int fb[256];
    const int tid = threadIdx.x;
    for (int j = tid; j < 257; j += kThreads) {
        A[j] = Ag[j];
        if (averages) averages[j] = A[j];
    }
    __syncthreads();
    const double qi = (A[tid] + A[tid + 1]) * 0.5;
    q[tid] = qi;
    // the largest magnitude (a maximum: exact in any order)
    double m = fabs(qi);
    for (int off = 32; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    const float v = m > 0.0 ? (float)(q[tid] / m) : 0.0f;
    vals[tid] = v;
    out->values[tid] = v;
    __syncthreads();
    if (tid < 255) {
        const float a = vals[tid], b = vals[tid + 1];
        const double mid = ((double)a + (double)b) / 2.0;   // the binary64 midpoint, as the encoder reads it
        const float t = ceil_f32(mid, fabsf(a) < fabsf(b));
        out->thr[tid] = t;
        fb[tid] = user_bucket(t);
    } else {
        out->thr[255] = INFINITY;
    }
    __syncthreads();
    // the bucket index: first[b] = #{k < 255 : fb[k] < b} (fb ascending), by a
    // lower-bound search per bucket
    for (int b = tid; b < kUserFirstBytes; b += kThreads) {
        uint32_t lo = 0;
        if (b <= kUserBuckets) {
            uint32_t len = 255;
            while (len != 0) {
                const uint32_t h = len >> 1;
                if (fb[lo + h] < b) {
                    lo += h + 1;
                    len -= h + 1;
                } else {
                    len = h;
                }
            }
        }
        out->first[b] = (uint8_t)lo;
    }
}

}  // namespace

hipError_t launch_chunk_quantiles(const void* x, int xdt, int64_t n, float* E, hipStream_t s)
{
    const int64_t nchunks = (n + kQuantileChunk - 1) / kQuantileChunk;
    if (nchunks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (xdt) {
    case DT_F32: return launch_kernel(k_chunk_quantiles<DT_F32>, (int)nchunks, s, x, n, nchunks, E);
    case DT_F16: return launch_kernel(k_chunk_quantiles<DT_F16>, (int)nchunks, s, x, n, nchunks, E);
    case DT_BF16: return launch_kernel(k_chunk_quantiles<DT_BF16>, (int)nchunks, s, x, n, nchunks, E);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantile_code(const float* E, int64_t nchunks, double* A, double* averages, UserCode* out,
                                hipStream_t s)
{
    hipError_t e = launch_kernel(k_quantile_means, 257, s, E, nchunks, A);
    if (e != hipSuccess) return e;
    return launch_kernel(k_quantile_code, 1, s, (const double*)A, averages, out);
}

}  // namespace qb
