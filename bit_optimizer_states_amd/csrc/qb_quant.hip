// qb_quant.hip -- block-wise quantize / dequantize kernels (8-bit dynamic code
// and 4-bit NF4 / FP4), with the nested quantization of the block absmax.
//
// Method: every block of B consecutive elements is scaled by its own absolute
// maximum and each scaled value is encoded as the nearest code entry, blocks
// independently (abstract of "8-bit Optimizers via Block-wise Quantization"
// quoted on "Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略",
// section 2); 4-bit codes are packed two per byte ("bitsandbytes - Quantização
// de LLM", section Etapa 1); the absmax may itself be quantized a second time
// ("Bitsandbytes", section İç içe nicelleştirme).
//
// Kernel shape (all kernels): persistent 256-thread workgroups stride over
// fixed-size tiles; the tables are staged into LDS once per workgroup.  A tile
// whose elements all lie below n takes unguarded 128/64/32-bit loads and
// stores; only the last tile is guarded element by element.
#include "qb_device.h"
#include "qb_launch.h"

namespace qb {

// ---------------------------------------------------------------------------
// tile geometry
// ---------------------------------------------------------------------------

// 8-bit quantize: chunks of 4 elements (16 bytes of fp32 in, one u32 of codes out).
template <int B>
struct Tile8 {
    static constexpr int EPT = B >= 1024 ? B / 256 : 4;   // elements per thread
    static constexpr int LPB = B / EPT;                   // lanes per block: 16 .. 256
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
// it.  `red` is this tile's half of a double-buffered LDS scratch: the barrier
// of the next tile orders the reuse, so one barrier per tile suffices.
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

__device__ __forceinline__ uint32_t bit_at(const uint32_t* q, int i)
{
    return (q[i >> 5] >> (i & 31)) & 1u;
}

// Mean = (sum_b bins[b] 2^b) 2^-149 / count, rounded once to nearest-even
// binary32.  Single thread.  count < 2^32.
__device__ float exact_mean_from_bins(const unsigned long long* bins, uint32_t count)
{
    constexpr int W = 6;                           // 384-bit accumulator, 64-bit words
    unsigned long long w[W] = {0, 0, 0, 0, 0, 0};
    for (int b = 0; b < 254; ++b) {
        const unsigned long long c = bins[b];
        if (!c) continue;
        const int q = b >> 6, s = b & 63;
        unsigned long long lo = c << s, hi = s ? (c >> (64 - s)) : 0ull;
        unsigned long long old = w[q];
        w[q] += lo;
        unsigned long long carry = hi + (w[q] < old ? 1ull : 0ull);
        for (int k = q + 1; k < W && carry; ++k) {
            old = w[k];
            w[k] += carry;
            carry = w[k] < old ? 1ull : 0ull;
        }
    }
    uint32_t limb[2 * W], quo[2 * W];
    for (int i = 0; i < W; ++i) {
        limb[2 * i] = (uint32_t)w[i];
        limb[2 * i + 1] = (uint32_t)(w[i] >> 32);
    }
    unsigned long long rem = 0;
    for (int i = 2 * W - 1; i >= 0; --i) {
        unsigned long long cur = (rem << 32) | limb[i];
        quo[i] = (uint32_t)(cur / count);
        rem = cur % count;
    }
    int h = -1;
    for (int i = 2 * W - 1; i >= 0 && h < 0; --i)
        if (quo[i]) h = i * 32 + 31 - __clz(quo[i]);
    if (h < 0) return (2 * rem > count) ? ffrom(1u) : 0.0f;   // below 2^-149; a tie goes to 0 (even)
    const int shift = h > 23 ? h - 23 : 0;
    uint32_t mant = 0;
    for (int k = 0; k < 24 && shift + k <= h; ++k) mant |= bit_at(quo, shift + k) << k;
    bool up;
    if (shift == 0) {
        up = (2 * rem > count) || (2 * rem == count && (mant & 1u));
    } else {
        const bool guard = bit_at(quo, shift - 1);
        bool sticky = rem != 0;
        for (int k = 0; k < shift - 1 && !sticky; ++k) sticky = bit_at(quo, k);
        up = guard && (sticky || (mant & 1u));
    }
    // fields: exponent = shift (+1 folded into the implicit bit of mant)
    return ffrom(((uint32_t)shift << 23) + mant + (up ? 1u : 0u));
}

// ---------------------------------------------------------------------------
// 8-bit dynamic-code quantize
// ---------------------------------------------------------------------------

// MODE: QM_PLAIN writes absmax; QM_DQ_FIRST also adds it to the exponent bins;
// QM_DQ_SECOND quantizes x - mean (the mean from the bins; written to *offset).
template <int B, int XDT, int MODE>
__global__ __launch_bounds__(256) void k_quant8(const void* __restrict__ x, int64_t n,
                                                uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                const QbTables* __restrict__ tab,
                                                unsigned long long* __restrict__ bins,
                                                float* __restrict__ offset, int64_t ntiles)
{
    using T = Tile8<B>;
    __shared__ uint2 s_lut[kDynLutN];
    __shared__ uint32_t s_red[2][4];
    __shared__ unsigned long long s_bins[MODE == QM_DQ_FIRST ? 256 : 1];
    __shared__ float s_mu;
    const int tid = threadIdx.x;
    const uint2* glut = reinterpret_cast<const uint2*>(tab->dyn8_lut);
    for (int i = tid; i < kDynLutN; i += kThreads) s_lut[i] = glut[i];
    if constexpr (MODE == QM_DQ_FIRST) s_bins[tid] = 0ull;
    if constexpr (MODE == QM_DQ_SECOND) {
        if (tid == 0) {
            const float mu = exact_mean_from_bins(bins, (uint32_t)n);
            s_mu = mu;
            if (blockIdx.x == 0) *offset = mu;
        }
    }
    __syncthreads();
    float mu = 0.0f;
    if constexpr (MODE == QM_DQ_SECOND) mu = s_mu;

    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nb = (n + B - 1) / B;
    int par = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1) {
        const int64_t blk = tile * T::BPT + bt;
        const int64_t bstart = blk * B;
        const bool full = (tile + 1) * T::ELEMS <= n;
        float v[T::EPT];
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) load4<XDT>(x, bstart + c * T::LPB * 4 + l * 4, &v[c * 4]);
            if constexpr (MODE == QM_DQ_SECOND) {
#pragma unroll
                for (int i = 0; i < T::EPT; ++i) v[i] = v[i] - mu;
            }
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                    float xv = 0.0f;
                    if (idx < n) {
                        xv = load1<XDT>(x, idx);
                        if constexpr (MODE == QM_DQ_SECOND) xv = xv - mu;
                    }
                    v[c * 4 + j] = xv;
                }
        }
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) mx = max(mx, fbits(v[i]) & 0x7FFFFFFFu);
        mx = block_max<T>(mx, s_red[par], tid);
        const float a = ffrom(mx);
        if (l == 0 && blk < nb) {
            absmax[blk] = a;
            if constexpr (MODE == QM_DQ_FIRST) bin_absmax(s_bins, mx);
        }

        const float r = a > 0.0f ? 1.0f / a : 0.0f;
        const bool fast = fast_div_ok(a);
        uint32_t packed[T::CH];
        if (__all(fast)) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                uint32_t w = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) w |= enc_dyn8(div_by_block(v[c * 4 + j], a, r), s_lut) << (8 * j);
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
                    w |= enc_dyn8(nv, s_lut) << (8 * j);
                }
                packed[c] = w;
            }
        }
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
                *reinterpret_cast<uint32_t*>(codes + bstart + c * T::LPB * 4 + l * 4) = packed[c];
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                    if (idx < n) codes[idx] = (uint8_t)(packed[c] >> (8 * j));
                }
        }
    }
    if constexpr (MODE == QM_DQ_FIRST) {
        __syncthreads();
        if (tid < 254 && s_bins[tid]) atomicAdd(&bins[tid], s_bins[tid]);
    }
}

// ---------------------------------------------------------------------------
// 4-bit (NF4 / FP4) quantize
// ---------------------------------------------------------------------------

template <int B, int XDT, int MODE>
__global__ __launch_bounds__(256) void k_quant4(const void* __restrict__ x, int64_t n,
                                                uint8_t* __restrict__ codes, float* __restrict__ absmax,
                                                const QbTables* __restrict__ tab, int code4,
                                                unsigned long long* __restrict__ bins, int64_t ntiles)
{
    using T = Tile4<B>;
    __shared__ uint2 s_lut[k4LutN];
    __shared__ uint32_t s_red[2][4];
    __shared__ unsigned long long s_bins[MODE == QM_DQ_FIRST ? 256 : 1];
    const int tid = threadIdx.x;
    const uint2* glut = reinterpret_cast<const uint2*>(code4 == 0 ? tab->nf4_lut : tab->fp4_lut);
    if (tid < k4LutN) s_lut[tid] = glut[tid];
    if constexpr (MODE == QM_DQ_FIRST) s_bins[tid] = 0ull;
    __syncthreads();

    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nb = (n + B - 1) / B;
    int par = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1) {
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
        uint32_t mx = 0;
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) mx = max(mx, fbits(v[i]) & 0x7FFFFFFFu);
        mx = block_max<T>(mx, s_red[par], tid);
        const float a = ffrom(mx);
        if (l == 0 && blk < nb) {
            absmax[blk] = a;
            if constexpr (MODE == QM_DQ_FIRST) bin_absmax(s_bins, mx);
        }

        const float r = a > 0.0f ? 1.0f / a : 0.0f;
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
            for (int c = 0; c < T::CH; ++c)
                *reinterpret_cast<uint32_t*>(codes + (bstart + c * T::LPB * 8 + l * 8) / 2) = packed[c];
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int64_t e0 = bstart + c * T::LPB * 8 + l * 8 + 2 * k;
                    if (e0 < n) {
                        uint32_t byte = (packed[c] >> (8 * k)) & 0xFFu;
                        if (e0 + 1 >= n) byte &= 0xF0u;        // odd n: the last low nibble is 0
                        codes[e0 / 2] = (uint8_t)byte;
                    }
                }
        }
    }
    if constexpr (MODE == QM_DQ_FIRST) {
        __syncthreads();
        if (tid < 254 && s_bins[tid]) atomicAdd(&bins[tid], s_bins[tid]);
    }
}

// ---------------------------------------------------------------------------
// dequantize
// ---------------------------------------------------------------------------

// Scale of block `blk`: its absmax, or with nesting dyn8[c2] * absmax2 + mean
// (two rounded binary32 operations).
template <bool DQ>
__device__ __forceinline__ float block_scale(int64_t blk, const float* __restrict__ absmax,
                                             const uint8_t* __restrict__ c2, const float* __restrict__ absmax2,
                                             int log2B2, float mu, const float* __restrict__ s_dyn)
{
    if constexpr (DQ) {
        const float prod = s_dyn[c2[blk]] * absmax2[blk >> log2B2];
        return prod + mu;
    } else {
        return absmax[blk];
    }
}

template <int YDT>
__device__ __forceinline__ void store4(void* __restrict__ y, int64_t i, const float* o)
{
    if constexpr (YDT == DT_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + i) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + i) = make_uint2(pack2<YDT>(o[0], o[1]), pack2<YDT>(o[2], o[3]));
    }
}

template <int YDT>
__device__ __forceinline__ void store8(void* __restrict__ y, int64_t i, const float* o)
{
    if constexpr (YDT == DT_F32) {
        store4<DT_F32>(y, i, o);
        store4<DT_F32>(y, i + 4, o + 4);
    } else {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + i) =
            make_uint4(pack2<YDT>(o[0], o[1]), pack2<YDT>(o[2], o[3]), pack2<YDT>(o[4], o[5]), pack2<YDT>(o[6], o[7]));
    }
}

constexpr int kDq8Units = 4;    // units of 4 codes per thread per tile
constexpr int kDq8Elems = kThreads * kDq8Units * 4;

template <int YDT, bool DQ>
__global__ __launch_bounds__(256) void k_dequant8(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                                  const uint8_t* __restrict__ c2, const float* __restrict__ absmax2,
                                                  const float* __restrict__ offset, int log2B, int log2B2, int64_t n,
                                                  void* __restrict__ y, const QbTables* __restrict__ tab,
                                                  int64_t ntiles)
{
    __shared__ float s_dyn[256];
    const int tid = threadIdx.x;
    s_dyn[tid] = tab->dyn8[tid];
    __syncthreads();
    const float mu = DQ ? *offset : 0.0f;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kDq8Elems;
        const bool full = base + kDq8Elems <= n;
        if (full) {
            uint32_t w[kDq8Units];
#pragma unroll
            for (int k = 0; k < kDq8Units; ++k)
                w[k] = *reinterpret_cast<const uint32_t*>(codes + base + k * kThreads * 4 + tid * 4);
#pragma unroll
            for (int k = 0; k < kDq8Units; ++k) {
                const int64_t e0 = base + k * kThreads * 4 + tid * 4;
                const float s = block_scale<DQ>(e0 >> log2B, absmax, c2, absmax2, log2B2, mu, s_dyn);
                float o[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = s_dyn[(w[k] >> (8 * j)) & 0xFFu] * s;
                store4<YDT>(y, e0, o);
            }
        } else {
            for (int k = 0; k < kDq8Units; ++k)
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = base + k * kThreads * 4 + tid * 4 + j;
                    if (idx < n) {
                        const float s = block_scale<DQ>(idx >> log2B, absmax, c2, absmax2, log2B2, mu, s_dyn);
                        store1<YDT>(y, idx, s_dyn[codes[idx]] * s);
                    }
                }
        }
    }
}

constexpr int kDq4Units = 4;    // units of 8 codes (one u32) per thread per tile
constexpr int kDq4Elems = kThreads * kDq4Units * 8;

template <int YDT, bool DQ>
__global__ __launch_bounds__(256) void k_dequant4(const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                                  const uint8_t* __restrict__ c2, const float* __restrict__ absmax2,
                                                  const float* __restrict__ offset, int log2B, int log2B2, int64_t n,
                                                  int code4, void* __restrict__ y, const QbTables* __restrict__ tab,
                                                  int64_t ntiles)
{
    __shared__ float2 s_pair[256];
    __shared__ float s_dyn[DQ ? 256 : 1];
    const int tid = threadIdx.x;
    const float* gp = &tab->pair[code4][0][0];
    s_pair[tid] = make_float2(gp[2 * tid], gp[2 * tid + 1]);
    if constexpr (DQ) s_dyn[tid] = tab->dyn8[tid];
    __syncthreads();
    const float mu = DQ ? *offset : 0.0f;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int64_t base = tile * kDq4Elems;
        const bool full = base + kDq4Elems <= n;
        if (full) {
            uint32_t w[kDq4Units];
#pragma unroll
            for (int k = 0; k < kDq4Units; ++k)
                w[k] = *reinterpret_cast<const uint32_t*>(codes + (base + k * kThreads * 8 + tid * 8) / 2);
#pragma unroll
            for (int k = 0; k < kDq4Units; ++k) {
                const int64_t e0 = base + k * kThreads * 8 + tid * 8;
                const float s = block_scale<DQ>(e0 >> log2B, absmax, c2, absmax2, log2B2, mu, s_dyn);
                float o[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float2 pr = s_pair[(w[k] >> (8 * j)) & 0xFFu];
                    o[2 * j] = pr.x * s;
                    o[2 * j + 1] = pr.y * s;
                }
                store8<YDT>(y, e0, o);
            }
        } else {
            for (int k = 0; k < kDq4Units; ++k)
                for (int j = 0; j < 8; ++j) {
                    const int64_t idx = base + k * kThreads * 8 + tid * 8 + j;
                    if (idx < n) {
                        const float s = block_scale<DQ>(idx >> log2B, absmax, c2, absmax2, log2B2, mu, s_dyn);
                        const float2 pr = s_pair[codes[idx / 2]];
                        store1<YDT>(y, idx, ((idx & 1) ? pr.y : pr.x) * s);
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

int ilog2(int v)
{
    int k = 0;
    while ((1 << k) < v) ++k;
    return k;
}

template <int B, int XDT, int MODE>
hipError_t quant8_as(const void* x, int64_t n, uint8_t* codes, float* absmax, const QbTables* tab,
                     unsigned long long* bins, float* offset, hipStream_t s)
{
    const int64_t ntiles = (n + Tile8<B>::ELEMS - 1) / Tile8<B>::ELEMS;
    auto kern = k_quant8<B, XDT, MODE>;
    return launch_kernel(kern, persistent_grid(kern, ntiles), s, x, n, codes, absmax, tab, bins, offset, ntiles);
}

template <int B, int MODE>
hipError_t quant8_dt(int xdt, const void* x, int64_t n, uint8_t* codes, float* absmax, const QbTables* tab,
                     unsigned long long* bins, float* offset, hipStream_t s)
{
    switch (xdt) {
    case DT_F32: return quant8_as<B, DT_F32, MODE>(x, n, codes, absmax, tab, bins, offset, s);
    case DT_F16: return quant8_as<B, DT_F16, MODE>(x, n, codes, absmax, tab, bins, offset, s);
    case DT_BF16: return quant8_as<B, DT_BF16, MODE>(x, n, codes, absmax, tab, bins, offset, s);
    default: return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t quant8_b(int B, int xdt, const void* x, int64_t n, uint8_t* codes, float* absmax, const QbTables* tab,
                    unsigned long long* bins, float* offset, hipStream_t s)
{
    switch (B) {
    case 64: return quant8_dt<64, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 128: return quant8_dt<128, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 256: return quant8_dt<256, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 512: return quant8_dt<512, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 1024: return quant8_dt<1024, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 2048: return quant8_dt<2048, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    case 4096: return quant8_dt<4096, MODE>(xdt, x, n, codes, absmax, tab, bins, offset, s);
    default: return hipErrorInvalidValue;
    }
}

template <int B, int XDT, int MODE>
hipError_t quant4_as(const void* x, int64_t n, int code4, uint8_t* codes, float* absmax, const QbTables* tab,
                     unsigned long long* bins, hipStream_t s)
{
    const int64_t ntiles = (n + Tile4<B>::ELEMS - 1) / Tile4<B>::ELEMS;
    auto kern = k_quant4<B, XDT, MODE>;
    return launch_kernel(kern, persistent_grid(kern, ntiles), s, x, n, codes, absmax, tab, code4, bins, ntiles);
}

template <int B, int MODE>
hipError_t quant4_dt(int xdt, const void* x, int64_t n, int code4, uint8_t* codes, float* absmax,
                     const QbTables* tab, unsigned long long* bins, hipStream_t s)
{
    switch (xdt) {
    case DT_F32: return quant4_as<B, DT_F32, MODE>(x, n, code4, codes, absmax, tab, bins, s);
    case DT_F16: return quant4_as<B, DT_F16, MODE>(x, n, code4, codes, absmax, tab, bins, s);
    case DT_BF16: return quant4_as<B, DT_BF16, MODE>(x, n, code4, codes, absmax, tab, bins, s);
    default: return hipErrorInvalidValue;
    }
}

template <int MODE>
hipError_t quant4_b(int B, int xdt, const void* x, int64_t n, int code4, uint8_t* codes, float* absmax,
                    const QbTables* tab, unsigned long long* bins, hipStream_t s)
{
    switch (B) {
    case 64: return quant4_dt<64, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 128: return quant4_dt<128, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 256: return quant4_dt<256, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 512: return quant4_dt<512, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 1024: return quant4_dt<1024, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 2048: return quant4_dt<2048, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    case 4096: return quant4_dt<4096, MODE>(xdt, x, n, code4, codes, absmax, tab, bins, s);
    default: return hipErrorInvalidValue;
    }
}

template <int YDT, bool DQ>
hipError_t dequant8_as(const uint8_t* codes, const float* absmax, const uint8_t* c2, const float* absmax2,
                       const float* offset, int B, int B2, int64_t n, void* y, const QbTables* tab, hipStream_t s)
{
    const int64_t ntiles = (n + kDq8Elems - 1) / kDq8Elems;
    auto kern = k_dequant8<YDT, DQ>;
    return launch_kernel(kern, persistent_grid(kern, ntiles), s, codes, absmax, c2, absmax2, offset, ilog2(B),
                         ilog2(B2), n, y, tab, ntiles);
}

template <int YDT, bool DQ>
hipError_t dequant4_as(const uint8_t* codes, const float* absmax, const uint8_t* c2, const float* absmax2,
                       const float* offset, int B, int B2, int64_t n, int code4, void* y, const QbTables* tab,
                       hipStream_t s)
{
    const int64_t ntiles = (n + kDq4Elems - 1) / kDq4Elems;
    auto kern = k_dequant4<YDT, DQ>;
    return launch_kernel(kern, persistent_grid(kern, ntiles), s, codes, absmax, c2, absmax2, offset, ilog2(B),
                         ilog2(B2), n, code4, y, tab, ntiles);
}

}  // namespace

hipError_t launch_quant8(const void* x, int xdt, int64_t n, int B, uint8_t* codes, float* absmax, int mode,
                         unsigned long long* bins, float* offset, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    switch (mode) {
    case QM_PLAIN: return quant8_b<QM_PLAIN>(B, xdt, x, n, codes, absmax, tab, bins, offset, s);
    case QM_DQ_FIRST: return quant8_b<QM_DQ_FIRST>(B, xdt, x, n, codes, absmax, tab, bins, offset, s);
    case QM_DQ_SECOND:
        // the second level always reads the fp32 absmax
        return quant8_b<QM_DQ_SECOND>(B, DT_F32, x, n, codes, absmax, tab, bins, offset, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quant4(const void* x, int xdt, int64_t n, int B, int code4, uint8_t* codes, float* absmax,
                         int mode, unsigned long long* bins, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (mode == QM_PLAIN) return quant4_b<QM_PLAIN>(B, xdt, x, n, code4, codes, absmax, tab, bins, s);
    if (mode == QM_DQ_FIRST) return quant4_b<QM_DQ_FIRST>(B, xdt, x, n, code4, codes, absmax, tab, bins, s);
    return hipErrorInvalidValue;
}

hipError_t launch_dequant8(const uint8_t* codes, const float* absmax, const uint8_t* c2, const float* absmax2,
                           const float* offset, int B, int B2, int64_t n, void* y, int ydt, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    const bool dq = c2 != nullptr;
    switch (ydt) {
    case DT_F32: return dq ? dequant8_as<DT_F32, true>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s)
                           : dequant8_as<DT_F32, false>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s);
    case DT_F16: return dq ? dequant8_as<DT_F16, true>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s)
                           : dequant8_as<DT_F16, false>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s);
    case DT_BF16: return dq ? dequant8_as<DT_BF16, true>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s)
                            : dequant8_as<DT_BF16, false>(codes, absmax, c2, absmax2, offset, B, B2, n, y, tab, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequant4(const uint8_t* codes, const float* absmax, const uint8_t* c2, const float* absmax2,
                           const float* offset, int B, int B2, int64_t n, int code4, void* y, int ydt,
                           hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    const bool dq = c2 != nullptr;
    switch (ydt) {
    case DT_F32: return dq ? dequant4_as<DT_F32, true>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s)
                           : dequant4_as<DT_F32, false>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s);
    case DT_F16: return dq ? dequant4_as<DT_F16, true>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s)
                           : dequant4_as<DT_F16, false>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s);
    case DT_BF16: return dq ? dequant4_as<DT_BF16, true>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s)
                            : dequant4_as<DT_BF16, false>(codes, absmax, c2, absmax2, offset, B, B2, n, code4, y, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qb
