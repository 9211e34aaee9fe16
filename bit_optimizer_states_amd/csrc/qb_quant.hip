// qb_quant.hip -- block-wise quantization kernels (8-bit dynamic code and 4-bit
// NF4 / FP4), with the nested quantization of the block absmax.
//
// Method: every block of B consecutive elements is scaled by its own absolute
// maximum and each scaled value is encoded as the nearest code entry, blocks
// independently (abstract of "8-bit Optimizers via Block-wise Quantization"
// quoted on "Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略",
// section 2); 4-bit codes are packed two per byte ("bitsandbytes - Quantização
// de LLM", section Etapa 1); the absmax may itself be quantized a second time
// ("Bitsandbytes", section İç içe nicelleştirme).
//
// Kernel shape: one 256-thread workgroup per tile, launched in tile order, so
// the HBM accesses of all resident workgroups form one narrow moving front
// (measured on MI355X: a copy reaches 6.2 TB/s this way against 4.6 TB/s for a
// persistent grid-stride loop).  Each workgroup issues its tile's loads before
// staging its small LDS tables, so the staging hides under the load latency.
// A tile whose elements all lie below n takes unguarded vector loads and
// stores; only the last tile is guarded element by element.  The first pass of
// a nested quantization is the exception: it strides persistently so that each
// workgroup flushes its exponent bins with few global atomics.
#include "qb_device.h"
#include "qb_launch.h"

namespace qb {

// ---------------------------------------------------------------------------
// tile geometry
// ---------------------------------------------------------------------------

// 8-bit quantize: chunks of 4 elements (16 bytes of fp32 in, one u32 of codes
// out); at least 8 elements per thread.
template <int B>
struct Tile8 {
    static constexpr int EPT = B >= 2048 ? B / 256 : 8;   // elements per thread
    static constexpr int LPB = B / EPT;                   // lanes per block: 8 .. 256
    static constexpr int BPT = kThreads / LPB;            // blocks per tile
    static constexpr int CH = EPT / 4;                    // chunks per thread
    static constexpr int ELEMS = kThreads * EPT;          // elements per tile
    static constexpr int WPB = LPB > 64 ? LPB / 64 : 1;   // waves per block
};

// 4-bit quantize: chunks of 8 elements (one u32 of packed codes out).
template <int B>
struct Tile4 {
    static constexpr int EPT = B >= 4096 ? B / 256 : 8;
    static constexpr int LPB = B / EPT;                   // 8 .. 256
    static constexpr int BPT = kThreads / LPB;
    static constexpr int CH = EPT / 8;
    static constexpr int ELEMS = kThreads * EPT;
    static constexpr int WPB = LPB > 64 ? LPB / 64 : 1;
};

// Block maximum of non-negative values (as bits); every lane of the block gets
// it.  `red` is a double-buffered LDS scratch half: with persistent loops the
// next tile's barrier orders its reuse, so one barrier per tile suffices.
template <class T>
__device__ __forceinline__ uint32_t block_max(uint32_t x, uint32_t* red, int tid)
{
    constexpr int L = T::LPB < 64 ? T::LPB : 64;
    x = lanes_max<L>(x);
    if constexpr (T::WPB > 1) {
        const int w = tid >> 6;
        if ((tid & 63) == 0) red[w] = x;
        __syncthreads();
        const int first = (w / T::WPB) * T::WPB;
        uint32_t y = 0;
#pragma unroll
        for (int i = 0; i < T::WPB; ++i) y = max(y, red[first + i]);
        x = y;
    }
    return x;
}

// ---------------------------------------------------------------------------
// exact mean of the absmax (nested quantization)
// ---------------------------------------------------------------------------

// Adds the block absmax a >= 0 to the exponent bins: a = M * 2^(e - 150) with a
// 24-bit integer M and e = max(biased exponent, 1); bin e-1 accumulates M, so
// the sum is exact and independent of order (integer atomics).
__device__ __forceinline__ void bin_absmax(unsigned long long* s_bins, uint32_t abits)
{
    const uint32_t e = abits >> 23;
    const uint32_t m = (abits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    if (m) atomicAdd(&s_bins[(e ? e : 1u) - 1u], (unsigned long long)m);
}

// Mean = S 2^-149 / count with S = sum_b c[b] 2^b (c[] in LDS, nonzero bins
// flagged in mask[4]), rounded once to nearest-even binary32.  One thread.
// S (< 2^320) is accumulated exactly; its top 96 bits W are divided by count
// (< 2^32) in three 64/32-bit steps.  With S = W 2^sh + R (R < 2^sh):
// S / count = Q 2^sh + (r 2^sh + R) / count, the last term below 2^sh and
// zero iff r == 0 and R == 0, so Q plus that sticky flag decide the rounding.
__device__ float mean_from_bins(const unsigned long long* c, const unsigned long long* mask, uint32_t count)
{
    unsigned long long w[6] = {0, 0, 0, 0, 0, 0};
    for (int q = 0; q < 4; ++q) {
        unsigned long long mk = mask[q];
        while (mk) {
            const int b = q * 64 + __ffsll((long long)mk) - 1;
            mk &= mk - 1;
            const unsigned long long cb = c[b];
            const int wi = b >> 6, s = b & 63;
            const unsigned long long lo = cb << s, hi = s ? (cb >> (64 - s)) : 0ull;
            unsigned long long old = w[wi];
            w[wi] += lo;
            unsigned long long carry = hi + (w[wi] < old ? 1ull : 0ull);
            for (int k = wi + 1; k < 6 && carry; ++k) {
                old = w[k];
                w[k] += carry;
                carry = w[k] < old ? 1ull : 0ull;
            }
        }
    }
    int top = 5;
    while (top >= 0 && w[top] == 0) --top;
    if (top < 0) return 0.0f;
    const int L = top * 64 + 63 - __clzll((long long)w[top]);   // top set bit of S
    const int sh = L > 95 ? L - 95 : 0;
    auto bits32 = [&](int pos) -> uint32_t {                     // bits [pos, pos+32) of S
        const int q = pos >> 6, r = pos & 63;
        unsigned long long v = q < 6 ? (w[q] >> r) : 0ull;
        if (r && q + 1 < 6) v |= w[q + 1] << (64 - r);
        return (uint32_t)v;
    };
    bool low_nz = false;                                          // R != 0
    for (int q = 0; q < 6 && q * 64 < sh; ++q) {
        const int nbits = sh - q * 64;
        const unsigned long long mk = nbits >= 64 ? ~0ull : ((1ull << nbits) - 1ull);
        if (w[q] & mk) low_nz = true;
    }
    const uint32_t l0 = bits32(sh), l1 = bits32(sh + 32), l2 = bits32(sh + 64);
    unsigned long long cur = l2;
    const unsigned long long q2 = cur / count;
    unsigned long long r = cur % count;
    cur = (r << 32) | l1;
    const unsigned long long q1 = cur / count;
    r = cur % count;
    cur = (r << 32) | l0;
    const unsigned long long q0 = cur / count;
    r = cur % count;
    const unsigned __int128 Q = ((unsigned __int128)q2 << 64) | ((unsigned __int128)q1 << 32) | q0;
    if (Q == 0) return (2 * r > count) ? ffrom(1u) : 0.0f;         // below 2^-149 (sh == 0 here)
    const unsigned long long qhi = (unsigned long long)(Q >> 64), qlo = (unsigned long long)Q;
    const int H = qhi ? 64 + 63 - __clzll((long long)qhi) : 63 - __clzll((long long)qlo);
    const int srel = H > 23 ? H - 23 : 0;
    const uint32_t mant = (uint32_t)(Q >> srel);
    bool up;
    if (srel == 0) {
        up = (2 * r > count) || (2 * r == count && (mant & 1u));
    } else {
        const bool guard = (uint32_t)(Q >> (srel - 1)) & 1u;
        const unsigned __int128 below = Q & ((((unsigned __int128)1) << (srel - 1)) - 1);
        const bool sticky = below != 0 || r != 0 || low_nz;
        up = guard && (sticky || (mant & 1u));
    }
    // binary32 fields: exponent (srel + sh), the implicit bit folded into mant
    return ffrom(((uint32_t)(srel + sh) << 23) + mant + (up ? 1u : 0u));
}

// Every workgroup of the nested second pass computes the mean itself: the
// bins are loaded in parallel (one per thread), one thread does the arithmetic.
__device__ __forceinline__ float exact_mean_wg(const unsigned long long* __restrict__ bins, uint32_t count, int tid)
{
    __shared__ unsigned long long s_c[256];
    __shared__ unsigned long long s_mask[4];
    __shared__ float s_mu;
    unsigned long long c = 0;
    if (tid < 254) {
#pragma unroll
        for (int k = 0; k < kBinCopies; ++k) c += bins[k * 256 + tid];
    }
    s_c[tid] = c;
    const unsigned long long mk = __ballot(c != 0ull);
    if ((tid & 63) == 0) s_mask[tid >> 6] = mk;
    __syncthreads();
    if (tid == 0) s_mu = mean_from_bins(s_c, s_mask, count);
    __syncthreads();
    return s_mu;
}

// ---------------------------------------------------------------------------
// 8-bit dynamic-code quantize
// ---------------------------------------------------------------------------

// One tile of the 8-bit quantizer.  MODE: QM_PLAIN writes absmax; QM_DQ_FIRST
// also bins it; QM_DQ_SECOND quantizes x - mu.
template <int B, int XDT, int MODE>
__device__ __forceinline__ void quant8_tile(int64_t tile, const void* __restrict__ x, int64_t n,
                                           uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                           float mu, unsigned long long* s_bins, uint32_t* red,
                                           const DynEncLds& enc, const QbTables* __restrict__ tab,
                                           DynEncLds* stage, int tid)
{
    using T = Tile8<B>;
    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nb = (n + B - 1) / B;
    const int64_t blk = tile * T::BPT + bt;
    const int64_t bstart = blk * B;
    const bool full = (tile + 1) * T::ELEMS <= n;
    float v[T::EPT];
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) load4<XDT>(x, bstart + c * T::LPB * 4 + l * 4, &v[c * 4]);
    } else {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                v[c * 4 + j] = idx < n ? load1<XDT>(x, idx) : 0.0f;
            }
    }
    if (stage) {            // one-tile launches: stage the tables while the loads fly
        stage_dyn_enc(*stage, tab, tid);
        __syncthreads();
    }
    if constexpr (MODE == QM_DQ_SECOND) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (full || bstart + c * T::LPB * 4 + l * 4 + j < n) v[c * 4 + j] = v[c * 4 + j] - mu;
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < T::EPT; ++i) mx = max(mx, fbits(v[i]) & 0x7FFFFFFFu);
    mx = block_max<T>(mx, red, tid);
    const float a = ffrom(mx);
    if (l == 0 && blk < nb) {
        gst<float>(absmax + blk, a);
        if constexpr (MODE == QM_DQ_FIRST) bin_absmax(s_bins, mx);
    }

    const float r = rcp_rn(a);            // used only where fast_div_ok(a)
    const bool fast = fast_div_ok(a);
    uint32_t packed[T::CH];
    if (__all(fast)) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) w |= enc_dyn8(div_by_block(v[c * 4 + j], a, r), enc) << (8 * j);
            packed[c] = w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xv = v[c * 4 + j];
                const float nv = fast ? div_by_block(xv, a, r) : (a > 0.0f ? xv / a : 0.0f);
                w |= enc_dyn8(nv, enc) << (8 * j);
            }
            packed[c] = w;
        }
    }
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) gst<uint32_t>(codes + bstart + c * T::LPB * 4 + l * 4, packed[c]);
    } else {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                if (idx < n) gst<uint8_t>(codes + idx, (uint8_t)(packed[c] >> (8 * j)));
            }
    }
}

// One workgroup per tile (QM_PLAIN, QM_DQ_SECOND).
template <int B, int XDT, int MODE>
__global__ __launch_bounds__(256) void k_quant8(const void* __restrict__ x, int64_t n,
                                                uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                const QbTables* __restrict__ tab,
                                                const unsigned long long* __restrict__ bins,
                                                float* __restrict__ offset)
{
    __shared__ DynEncLds s_enc;
    __shared__ uint32_t s_red[4];
    const int tid = threadIdx.x;
    float mu = 0.0f;
    if constexpr (MODE == QM_DQ_SECOND) {
        mu = exact_mean_wg(bins, (uint32_t)n, tid);
        if (blockIdx.x == 0 && tid == 0) gst<float>(offset, mu);
    }
    quant8_tile<B, XDT, MODE>(blockIdx.x, x, n, codes, absmax, mu, nullptr, s_red, s_enc, tab, &s_enc, tid);
}

// Persistent grid-stride variant for the first pass of a nested quantization.
template <int B, int XDT>
__global__ __launch_bounds__(256) void k_quant8_binned(const void* __restrict__ x, int64_t n,
                                                       uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                       const QbTables* __restrict__ tab,
                                                       unsigned long long* __restrict__ bins, int64_t ntiles)
{
    __shared__ DynEncLds s_enc;
    __shared__ uint32_t s_red[2][4];
    __shared__ unsigned long long s_bins[256];
    const int tid = threadIdx.x;
    stage_dyn_enc(s_enc, tab, tid);
    s_bins[tid] = 0ull;
    __syncthreads();
    int par = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1)
        quant8_tile<B, XDT, QM_DQ_FIRST>(tile, x, n, codes, absmax, 0.0f, s_bins, s_red[par], s_enc, tab, nullptr, tid);
    __syncthreads();
    if (tid < 254 && s_bins[tid]) atomicAdd(&bins[(blockIdx.x % kBinCopies) * 256 + tid], s_bins[tid]);
}

// ---------------------------------------------------------------------------
// 4-bit (NF4 / FP4) quantize
// ---------------------------------------------------------------------------

template <int B, int XDT, int MODE>
__device__ __forceinline__ void quant4_tile(int64_t tile, const void* __restrict__ x, int64_t n,
                                           uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                           unsigned long long* s_bins, uint32_t* red, uint2* s_lut,
                                           const uint2* __restrict__ glut, bool stage, int tid)
{
    using T = Tile4<B>;
    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nb = (n + B - 1) / B;
    const int64_t blk = tile * T::BPT + bt;
    const int64_t bstart = blk * B;
    const bool full = (tile + 1) * T::ELEMS <= n;
    float v[T::EPT];
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) load8<XDT>(x, bstart + c * T::LPB * 8 + l * 8, &v[c * 8]);
    } else {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t idx = bstart + c * T::LPB * 8 + l * 8 + j;
                v[c * 8 + j] = idx < n ? load1<XDT>(x, idx) : 0.0f;
            }
    }
    if (stage) {
        if (tid < k4LutN) s_lut[tid] = glut[tid];
        __syncthreads();
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < T::EPT; ++i) mx = max(mx, fbits(v[i]) & 0x7FFFFFFFu);
    mx = block_max<T>(mx, red, tid);
    const float a = ffrom(mx);
    if (l == 0 && blk < nb) {
        gst<float>(absmax + blk, a);
        if constexpr (MODE == QM_DQ_FIRST) bin_absmax(s_bins, mx);
    }

    const float r = rcp_rn(a);            // used only where fast_div_ok(a)
    const bool fast = fast_div_ok(a);
    const bool all_fast = __all(fast);
    uint32_t packed[T::CH];
#pragma unroll
    for (int c = 0; c < T::CH; ++c) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float n0 = v[c * 8 + 2 * k], n1 = v[c * 8 + 2 * k + 1];
            if (all_fast) {
                n0 = div_by_block(n0, a, r);
                n1 = div_by_block(n1, a, r);
            } else {
                n0 = fast ? div_by_block(n0, a, r) : (a > 0.0f ? n0 / a : 0.0f);
                n1 = fast ? div_by_block(n1, a, r) : (a > 0.0f ? n1 / a : 0.0f);
            }
            const uint32_t byte = (enc_4bit(n0, s_lut) << 4) | enc_4bit(n1, s_lut);
            w |= byte << (8 * k);
        }
        packed[c] = w;
    }
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) gst<uint32_t>(codes + (bstart + c * T::LPB * 8 + l * 8) / 2, packed[c]);
    } else {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t e0 = bstart + c * T::LPB * 8 + l * 8 + 2 * k;
                if (e0 < n) {
                    uint32_t byte = (packed[c] >> (8 * k)) & 0xFFu;
                    if (e0 + 1 >= n) byte &= 0xF0u;        // odd n: the last low nibble is 0
                    gst<uint8_t>(codes + e0 / 2, (uint8_t)byte);
                }
            }
    }
}

template <int B, int XDT>
__global__ __launch_bounds__(256) void k_quant4(const void* __restrict__ x, int64_t n, uint8_t* __restrict__ codes,
                                                float* __restrict__ absmax, const QbTables* __restrict__ tab,
                                                int code4)
{
    __shared__ uint2 s_lut[k4LutN];
    __shared__ uint32_t s_red[4];
    const uint2* glut = reinterpret_cast<const uint2*>(code4 == 0 ? tab->nf4_lut : tab->fp4_lut);
    quant4_tile<B, XDT, QM_PLAIN>(blockIdx.x, x, n, codes, absmax, nullptr, s_red, s_lut, glut, true, threadIdx.x);
}

template <int B, int XDT>
__global__ __launch_bounds__(256) void k_quant4_binned(const void* __restrict__ x, int64_t n,
                                                       uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                       const QbTables* __restrict__ tab, int code4,
                                                       unsigned long long* __restrict__ bins, int64_t ntiles)
{
    __shared__ uint2 s_lut[k4LutN];
    __shared__ uint32_t s_red[2][4];
    __shared__ unsigned long long s_bins[256];
    const int tid = threadIdx.x;
    const uint2* glut = reinterpret_cast<const uint2*>(code4 == 0 ? tab->nf4_lut : tab->fp4_lut);
    if (tid < k4LutN) s_lut[tid] = glut[tid];
    s_bins[tid] = 0ull;
    __syncthreads();
    int par = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1)
        quant4_tile<B, XDT, QM_DQ_FIRST>(tile, x, n, codes, absmax, s_bins, s_red[par], s_lut, glut, false, tid);
    __syncthreads();
    if (tid < 254 && s_bins[tid]) atomicAdd(&bins[(blockIdx.x % kBinCopies) * 256 + tid], s_bins[tid]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

template <int B, int XDT>
hipError_t quant8_as(int mode, const void* x, int64_t n, uint8_t* codes, float* absmax, const QbTables* tab,
                     unsigned long long* bins, float* offset, hipStream_t s)
{
    const int64_t ntiles = (n + Tile8<B>::ELEMS - 1) / Tile8<B>::ELEMS;
    if (mode == QM_DQ_FIRST) {
        auto kern = k_quant8_binned<B, XDT>;
        return launch_kernel(kern, persistent_grid(kern, ntiles), s, x, n, codes, absmax, tab, bins, ntiles);
    }
    if (mode == QM_DQ_SECOND) {
        auto kern = k_quant8<B, XDT, QM_DQ_SECOND>;
        return launch_kernel(kern, (int)ntiles, s, x, n, codes, absmax, tab, bins, offset);
    }
    auto kern = k_quant8<B, XDT, QM_PLAIN>;
    return launch_kernel(kern, (int)ntiles, s, x, n, codes, absmax, tab, bins, offset);
}

template <int B>
hipError_t quant8_dt(int mode, int xdt, const void* x, int64_t n, uint8_t* codes, float* absmax, const QbTables* tab,
                     unsigned long long* bins, float* offset, hipStream_t s)
{
    switch (xdt) {
    case DT_F32: return quant8_as<B, DT_F32>(mode, x, n, codes, absmax, tab, bins, offset, s);
    case DT_F16: return quant8_as<B, DT_F16>(mode, x, n, codes, absmax, tab, bins, offset, s);
    case DT_BF16: return quant8_as<B, DT_BF16>(mode, x, n, codes, absmax, tab, bins, offset, s);
    default: return hipErrorInvalidValue;
    }
}

template <int B, int XDT>
hipError_t quant4_as(int mode, const void* x, int64_t n, int code4, uint8_t* codes, float* absmax,
                     const QbTables* tab, unsigned long long* bins, hipStream_t s)
{
    const int64_t ntiles = (n + Tile4<B>::ELEMS - 1) / Tile4<B>::ELEMS;
    if (mode == QM_DQ_FIRST) {
        auto kern = k_quant4_binned<B, XDT>;
        return launch_kernel(kern, persistent_grid(kern, ntiles), s, x, n, codes, absmax, tab, code4, bins, ntiles);
    }
    auto kern = k_quant4<B, XDT>;
    return launch_kernel(kern, (int)ntiles, s, x, n, codes, absmax, tab, code4);
}

template <int B>
hipError_t quant4_dt(int mode, int xdt, const void* x, int64_t n, int code4, uint8_t* codes, float* absmax,
                     const QbTables* tab, unsigned long long* bins, hipStream_t s)
{
    switch (xdt) {
    case DT_F32: return quant4_as<B, DT_F32>(mode, x, n, code4, codes, absmax, tab, bins, s);
    case DT_F16: return quant4_as<B, DT_F16>(mode, x, n, code4, codes, absmax, tab, bins, s);
    case DT_BF16: return quant4_as<B, DT_BF16>(mode, x, n, code4, codes, absmax, tab, bins, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

#define QB_SWITCH_B(B, CALL)                           \
    switch (B) {                                       \
    case 64: { constexpr int kB = 64; return CALL; }     \
    case 128: { constexpr int kB = 128; return CALL; }   \
    case 256: { constexpr int kB = 256; return CALL; }   \
    case 512: { constexpr int kB = 512; return CALL; }   \
    case 1024: { constexpr int kB = 1024; return CALL; } \
    case 2048: { constexpr int kB = 2048; return CALL; } \
    case 4096: { constexpr int kB = 4096; return CALL; } \
    default: return hipErrorInvalidValue;              \
    }

hipError_t launch_quant8(const void* x, int xdt, int64_t n, int B, uint8_t* codes, float* absmax, int mode,
                         unsigned long long* bins, float* offset, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (mode == QM_DQ_SECOND) xdt = DT_F32;     // the second level reads the fp32 absmax
    QB_SWITCH_B(B, quant8_dt<kB>(mode, xdt, x, n, codes, absmax, tab, bins, offset, s));
}

hipError_t launch_quant4(const void* x, int xdt, int64_t n, int B, int code4, uint8_t* codes, float* absmax,
                         int mode, unsigned long long* bins, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (mode != QM_PLAIN && mode != QM_DQ_FIRST) return hipErrorInvalidValue;
    QB_SWITCH_B(B, quant4_dt<kB>(mode, xdt, x, n, code4, codes, absmax, tab, bins, s));
}

}  // namespace qb
