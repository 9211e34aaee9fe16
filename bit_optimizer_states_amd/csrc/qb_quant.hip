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
// Kernel shape: one 256-thread workgroup per tile of 4096 elements (8192 for
// 4-bit codes), launched in
// tile order, so the HBM accesses of all resident workgroups form one narrow
// moving front (measured on MI355X: a copy reaches 6.2 TB/s this way against
// 4.6 TB/s for a persistent grid-stride loop).  A tile is R sub-tiles of
// 256 x EPT elements; a thread owns EPT elements of one block in every
// sub-tile (LPB lanes share a block).  Each workgroup issues all its loads
// before staging its LDS tables, so the staging hides under the load latency.
// A tile whose elements all lie below n takes unguarded vector loads and
// stores; only the last tile of a tensor is guarded element by element.
//
// Nested quantization takes four launches: clear the exponent bins, quantize
// (the fp32 absmax goes to a workspace and into the bins), compute the exact
// mean of the absmax from the bins, quantize absmax - mean with the dynamic
// code.  Many tensors go in one launch per step: tiles of all tensors are
// numbered in one range and a workgroup finds its tensor through the coarse
// bucket index.
#include <type_traits>

#include "qb_device.h"

namespace qb {

// XCD-contiguous tile order (tile_of) for grouped launches.
#ifndef QB_Q_MULTI_REMAP
#define QB_Q_MULTI_REMAP 1
#endif

// ---------------------------------------------------------------------------
// tile geometry
// ---------------------------------------------------------------------------

// BITS 8: chunks of 4 elements (one u32 of codes); BITS 4: chunks of 8 (one
// u32 of packed codes).  At least 8 elements per thread and sub-tile.
template <int BITS, int B>
struct QGeo {
    static constexpr int CW = BITS == 8 ? 4 : 8;                      // elements per chunk
    static constexpr int EPT = B / kThreads >= 8 ? B / kThreads : 8;  // elements per thread and sub-tile
    static constexpr int LPB = B / EPT;                               // lanes per block: 8 .. 256
    static constexpr int BPS = kThreads / LPB;                        // blocks per sub-tile
    static constexpr int CH = EPT / CW;                               // chunks per thread
    static constexpr int SUB = kThreads * EPT;                        // elements per sub-tile
    static constexpr int ELEMS = (int)quant_tile_elems(B, BITS);      // elements per tile
    static constexpr int R = ELEMS / SUB;                             // sub-tiles per tile
    static constexpr int WPB = LPB > 64 ? LPB / 64 : 1;               // waves per block
    static_assert(R >= 1 && ELEMS == SUB * R && EPT % CW == 0 && LPB <= kThreads, "quantize tile geometry");
};

// ---------------------------------------------------------------------------
// reductions and the exact mean
// ---------------------------------------------------------------------------

// Block maximum of non-negative values (as bits); every lane of the block gets
// it.  `red` is LDS scratch of its own per call site (no reuse, so one barrier
// per call suffices).
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
// quantize kernel
// ---------------------------------------------------------------------------

struct Lut4Lds {
    uint2 e[k4LutN];
};

// CW consecutive elements of dtype DT at element offset e from a uniform base.
template <int DT, int CW>
__device__ __forceinline__ void load_chunk(const void* base, uint32_t e, float* v)
{
    if constexpr (CW == 4) load4o<DT>(base, e, v);
    else load8o<DT>(base, e, v);
}

// One tile.  SECOND: the input is the fp32 absmax of a first pass and the
// tensor's mean (offset[0], written by k_dq_mean) is subtracted first.  With
// bins != nullptr (first pass of a nested quantization) every block absmax is
// also added to the tensor's exponent bins.
// USER: 8-bit codes of a user code (`user`: thresholds and their bucket index) instead of
// the dynamic code.
template <int BITS, int B, int XDT, bool SECOND, bool MULTI, bool USER = false>
__global__ __launch_bounds__(kThreads) void k_quant(QuantDesc single, TileMap<QuantDesc> map,
                                                   unsigned long long* __restrict__ bins,
                                                   const QbTables* __restrict__ tab, int code4,
                                                   const UserCode* __restrict__ user)
{
    static_assert(!USER || (BITS == 8 && !SECOND), "user codes are 8-bit, first pass only");
    using G = QGeo<BITS, B>;
    using EncLds = std::conditional_t<USER, UserEncLds, std::conditional_t<BITS == 8, DynEncLds, Lut4Lds>>;
    __shared__ EncLds s_enc;
    __shared__ uint32_t s_red[G::R][4];
    __shared__ unsigned long long s_bins[256];
    const int tid = threadIdx.x;
    const int64_t tile = tile_of<MULTI && QB_Q_MULTI_REMAP>(blockIdx.x, gridDim.x);

    QuantDesc d;
    int64_t lt;
    int ti;
    if constexpr (MULTI) {
        ti = find_tensor(map, tile);
        d = map.descs[ti];
        lt = tile - d.tile_begin;
    } else {
        ti = 0;
        d = single;
        lt = tile;
    }
    const int64_t n = d.n;
    const int64_t tbase = lt * G::ELEMS;                  // first element of the tile
    const bool full = tbase + G::ELEMS <= n;
    const int64_t rem = n - tbase;                        // elements of the tensor from the tile start
    const int bt = tid / G::LPB, l = tid % G::LPB;
    const void* const xt = static_cast<const char*>(d.x) + tbase * (XDT == DT_F32 ? 4 : 2);

    // loads of every sub-tile first.  RAW (4-bit codes of fp16 input): the
    // halves stay packed two per word; the block maximum is taken on them
    // with packed fp16 operations and the division reads them through
    // mixed-precision fused multiply-adds, so no element is converted.
    constexpr bool RAW = BITS == 4 && XDT == DT_F16 && !SECOND;
    float v[RAW ? 1 : G::R][RAW ? 1 : G::EPT];
    uint32_t hw[RAW ? G::R : 1][RAW ? G::EPT / 2 : 1];   // element 2i in the low half of word i
#pragma unroll
    for (int r = 0; r < G::R; ++r) {
        const uint32_t e0 = (uint32_t)((r * G::BPS + bt) * B + l * G::CW);   // chunk 0 of this thread
        if constexpr (RAW) {
#pragma unroll
            for (int c = 0; c < G::CH; ++c) {
                const uint32_t ec = e0 + c * G::LPB * G::CW;
                if (full) {
                    const u32x4 q = gldo<u32x4>(xt, ec * 2u);
                    hw[r][c * 4] = q.x;
                    hw[r][c * 4 + 1] = q.y;
                    hw[r][c * 4 + 2] = q.z;
                    hw[r][c * 4 + 3] = q.w;
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t e = ec + 2 * k;
                        const uint32_t lo = (int64_t)e < rem ? gld<uint16_t>(static_cast<const uint16_t*>(xt) + e) : 0u;
                        const uint32_t hi =
                            (int64_t)e + 1 < rem ? gld<uint16_t>(static_cast<const uint16_t*>(xt) + e + 1) : 0u;
                        hw[r][c * 4 + k] = lo | (hi << 16);
                    }
                }
            }
        } else if (full) {
#pragma unroll
            for (int c = 0; c < G::CH; ++c) load_chunk<XDT, G::CW>(xt, e0 + c * G::LPB * G::CW, &v[r][c * G::CW]);
        } else {
#pragma unroll
            for (int c = 0; c < G::CH; ++c)
#pragma unroll
                for (int j = 0; j < G::CW; ++j) {
                    const uint32_t e = e0 + c * G::LPB * G::CW + j;
                    v[r][c * G::CW + j] = (int64_t)e < rem ? load1<XDT>(xt, e) : 0.0f;
                }
        }
    }
    const bool binning = !SECOND && bins != nullptr;
    float mu = 0.0f;
    if constexpr (SECOND) mu = gld<float>(d.offset);
    if constexpr (USER) {
        stage_user_enc(s_enc, user, tid);
    } else if constexpr (BITS == 8) {
        stage_dyn_enc(s_enc, tab, tid);
    } else {
        const uint2* glut = reinterpret_cast<const uint2*>(code4 == 0 ? tab->nf4_lut : tab->fp4_lut);
        if (tid < k4LutN) s_enc.e[tid] = glut[tid];
    }
    if (binning) s_bins[tid] = 0ull;
    __syncthreads();

    const int64_t nb = (n + B - 1) / B;
    const int64_t blk0 = tbase / B;                       // a tile holds whole blocks
    uint32_t packed[G::R][G::CH];
#pragma unroll
    for (int r = 0; r < G::R; ++r) {
        float* const vr = v[RAW ? 0 : r];
        const int64_t blk = blk0 + r * G::BPS + bt;
        if constexpr (SECOND) {
            const uint32_t e0 = (uint32_t)((r * G::BPS + bt) * B + l * G::CW);
#pragma unroll
            for (int c = 0; c < G::CH; ++c)
#pragma unroll
                for (int j = 0; j < G::CW; ++j)
                    if (full || (int64_t)(e0 + c * G::LPB * G::CW + j) < rem) vr[c * G::CW + j] = vr[c * G::CW + j] - mu;
        }
        // max of |x| as a float max with the absolute-value operand modifier:
        // one instruction per element, equal to the max of the magnitude bits
        // for finite inputs (measured 2% faster on the 7B NF4 sweep than an
        // integer max of masked bits)
        float mf = 0.0f;
        if constexpr (RAW) {
            // |x| of both halves (sign bits cleared), then a packed 16-bit
            // integer max: for finite inputs the magnitudes order as integers
            u16x2 m2 = {0, 0};
#pragma unroll
            for (int i = 0; i < G::EPT / 2; ++i)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, hw[r][i] & 0x7FFF7FFFu));
            mf = (float)__builtin_bit_cast(_Float16, m2.x > m2.y ? m2.x : m2.y);
        } else {
#pragma unroll
            for (int i = 0; i < G::EPT; ++i) mf = __builtin_fmaxf(mf, __builtin_fabsf(vr[i]));
        }
        uint32_t mx = fbits(mf);
        mx = block_max<G>(mx, s_red[r], tid);
        const float a = ffrom(mx);
        if (l == 0 && blk < nb) {
            gst<float>(d.absmax + blk, a);
            if (binning) bin_absmax(s_bins, mx);
        }
        const float rc = rcp_rn(a);                      // used only where fast_div_ok(a)
        const bool fast = fast_div_ok(a);
        float nv[G::EPT];
        if constexpr (RAW) {
            if (__all(fast)) {
#pragma unroll
                for (int i = 0; i < G::EPT / 2; ++i) {
                    const h16x2 x2 = __builtin_bit_cast(h16x2, hw[r][i]);
                    nv[2 * i] = div_by_block_h(x2.x, a, rc);
                    nv[2 * i + 1] = div_by_block_h(x2.y, a, rc);
                }
            } else {
#pragma unroll
                for (int i = 0; i < G::EPT / 2; ++i) {
                    const h16x2 x2 = __builtin_bit_cast(h16x2, hw[r][i]);
                    nv[2 * i] = normalize_by_block((float)x2.x, a, rc, fast);
                    nv[2 * i + 1] = normalize_by_block((float)x2.y, a, rc, fast);
                }
            }
        } else if (__all(fast)) {                        // the usual case: one straight-line pass
#pragma unroll
            for (int i = 0; i < G::EPT; ++i) nv[i] = div_by_block(vr[i], a, rc);
        } else {
#pragma unroll
            for (int i = 0; i < G::EPT; ++i) nv[i] = normalize_by_block(vr[i], a, rc, fast);
        }
#pragma unroll
        for (int c = 0; c < G::CH; ++c) {
            uint32_t w = 0;
            if constexpr (BITS == 8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (USER) w |= enc_user(nv[c * 4 + j], s_enc) << (8 * j);
                    else w |= enc_dyn8(nv[c * 4 + j], s_enc) << (8 * j);
                }
            } else if (code4 == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w |= ((enc_nf4(nv[c * 8 + 2 * k], s_enc.e) << 4) | enc_nf4(nv[c * 8 + 2 * k + 1], s_enc.e))
                         << (8 * k);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w |= ((enc_fp4(nv[c * 8 + 2 * k], s_enc.e) << 4) | enc_fp4(nv[c * 8 + 2 * k + 1], s_enc.e))
                         << (8 * k);
            }
            packed[r][c] = w;
        }
    }

    // codes: one u32 per chunk (4 codes of 8 bits or 8 of 4 bits)
    uint8_t* const ct = d.codes + (tbase * BITS) / 8;
#pragma unroll
    for (int r = 0; r < G::R; ++r) {
        const uint32_t e0 = (uint32_t)((r * G::BPS + bt) * B + l * G::CW);
        if (full) {
#pragma unroll
            for (int c = 0; c < G::CH; ++c)
                gsto<uint32_t>(ct, (e0 + c * G::LPB * G::CW) * BITS / 8, packed[r][c]);
        } else {
#pragma unroll
            for (int c = 0; c < G::CH; ++c) {
                const uint32_t ec = e0 + c * G::LPB * G::CW;
                if constexpr (BITS == 8) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if ((int64_t)(ec + j) < rem) gst<uint8_t>(ct + ec + j, (uint8_t)(packed[r][c] >> (8 * j)));
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t e = ec + 2 * k;
                        if ((int64_t)e < rem) {
                            uint32_t byte = (packed[r][c] >> (8 * k)) & 0xFFu;
                            if ((int64_t)e + 1 >= rem) byte &= 0xF0u;   // odd n: the last low nibble is 0
                            gst<uint8_t>(ct + e / 2, (uint8_t)byte);
                        }
                    }
                }
            }
        }
    }

    if (binning) {
        __syncthreads();
        unsigned long long* const tb = bins + (size_t)ti * kBinWords + (blockIdx.x % kBinCopies) * 256;
        if (tid < 254 && s_bins[tid]) atomicAdd(&tb[tid], s_bins[tid]);
    }
}

// Exact mean of each tensor's absmax from its bins into offset[0]; one
// workgroup per tensor (descriptors of the second pass: n = absmax count).
template <bool MULTI>
__global__ __launch_bounds__(kThreads) void k_dq_mean(QuantDesc single, TileMap<QuantDesc> map,
                                                     const unsigned long long* __restrict__ bins)
{
    const int ti = MULTI ? (int)blockIdx.x : 0;
    const QuantDesc d = MULTI ? map.descs[ti] : single;
    const float mu = exact_mean_wg(bins + (size_t)ti * kBinWords, (uint32_t)d.n, threadIdx.x);
    if (threadIdx.x == 0) gst<float>(d.offset, mu);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

namespace {

template <int BITS, int B, int XDT, bool SECOND>
hipError_t quant_as(const QuantDesc& single, const TileMap<QuantDesc>* map, int64_t ntiles,
                    unsigned long long* bins, const QbTables* tab, int code4, hipStream_t s)
{
    if (map)
        return launch_kernel(k_quant<BITS, B, XDT, SECOND, true>, (int)ntiles, s, single, *map, bins, tab, code4,
                             (const UserCode*)nullptr);
    return launch_kernel(k_quant<BITS, B, XDT, SECOND, false>, (int)ntiles, s, single, TileMap<QuantDesc>{}, bins,
                         tab, code4, (const UserCode*)nullptr);
}

template <int BITS, int B>
hipError_t quant_x(int xdt, bool second, const QuantDesc& single, const TileMap<QuantDesc>* map, int64_t ntiles,
                   unsigned long long* bins, const QbTables* tab, int code4, hipStream_t s)
{
    if (second) {
        if constexpr (BITS == 8) return quant_as<8, B, DT_F32, true>(single, map, ntiles, nullptr, tab, 0, s);
        return hipErrorInvalidValue;
    }
    switch (xdt) {
    case DT_F32: return quant_as<BITS, B, DT_F32, false>(single, map, ntiles, bins, tab, code4, s);
    case DT_F16: return quant_as<BITS, B, DT_F16, false>(single, map, ntiles, bins, tab, code4, s);
    case DT_BF16: return quant_as<BITS, B, DT_BF16, false>(single, map, ntiles, bins, tab, code4, s);
    default: return hipErrorInvalidValue;
    }
}

template <int BITS>
hipError_t quant_b(int B, int xdt, bool second, const QuantDesc& single, const TileMap<QuantDesc>* map,
                   int64_t ntiles, unsigned long long* bins, const QbTables* tab, int code4, hipStream_t s)
{
    switch (B) {
    case 64: return quant_x<BITS, 64>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 128: return quant_x<BITS, 128>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 256: return quant_x<BITS, 256>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 512: return quant_x<BITS, 512>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 1024: return quant_x<BITS, 1024>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 2048: return quant_x<BITS, 2048>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    case 4096: return quant_x<BITS, 4096>(xdt, second, single, map, ntiles, bins, tab, code4, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quant(const QuantDesc& single, const TileMap<QuantDesc>* map, int64_t ntiles, int bits, int code4,
                        int B, int xdt, bool second, unsigned long long* bins, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (ntiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (bits == 8) return quant_b<8>(B, xdt, second, single, map, ntiles, bins, tab, code4, s);
    if (bits == 4 && !second) return quant_b<4>(B, xdt, false, single, map, ntiles, bins, tab, code4, s);
    return hipErrorInvalidValue;
}

namespace {

template <int B, int XDT>
hipError_t quant_user_as(const QuantDesc& d, int64_t ntiles, const UserCode* code, hipStream_t s)
{
    return launch_kernel(k_quant<8, B, XDT, false, false, true>, (int)ntiles, s, d, TileMap<QuantDesc>{},
                         (unsigned long long*)nullptr, (const QbTables*)nullptr, 0, code);
}

template <int B>
hipError_t quant_user_x(int xdt, const QuantDesc& d, int64_t ntiles, const UserCode* code, hipStream_t s)
{
    switch (xdt) {
    case DT_F32: return quant_user_as<B, DT_F32>(d, ntiles, code, s);
    case DT_F16: return quant_user_as<B, DT_F16>(d, ntiles, code, s);
    case DT_BF16: return quant_user_as<B, DT_BF16>(d, ntiles, code, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_quant_user(const QuantDesc& d, int64_t ntiles, int B, int xdt, const UserCode* code, hipStream_t s)
{
    if (ntiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (B) {
    case 64: return quant_user_x<64>(xdt, d, ntiles, code, s);
    case 128: return quant_user_x<128>(xdt, d, ntiles, code, s);
    case 256: return quant_user_x<256>(xdt, d, ntiles, code, s);
    case 512: return quant_user_x<512>(xdt, d, ntiles, code, s);
    case 1024: return quant_user_x<1024>(xdt, d, ntiles, code, s);
    case 2048: return quant_user_x<2048>(xdt, d, ntiles, code, s);
    case 4096: return quant_user_x<4096>(xdt, d, ntiles, code, s);
    default: return hipErrorInvalidValue;
    }
}

namespace {

// The normalized values of block-wise quantization, one element per thread:
// out[i] = x[i] / absmax[i / B] through the quantize kernels' own quotient
// (normalize_by_block with the block's rcp_rn and range test).  The
// correction step turns a quotient -0 into +0 (the encoders take both to the
// code of 0.0); here a zero quotient takes the sign of x, as IEEE division
// gives it.
template <int XDT>
__global__ __launch_bounds__(kThreads) void k_normalize(const void* __restrict__ x, int64_t n,
                                                        const float* __restrict__ absmax, int64_t B,
                                                        float* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const float a = absmax[i / B];
    const float xv = load1<XDT>(x, i);
    const float nv = normalize_by_block(xv, a, rcp_rn(a), fast_div_ok(a));
    out[i] = a > 0.0f ? __builtin_copysignf(nv, xv) : nv;
}

}  // namespace

hipError_t launch_normalize(const void* x, int xdt, int64_t n, const float* absmax, int64_t B, float* out,
                            hipStream_t s)
{
    const int64_t grid = (n + kThreads - 1) / kThreads;
    if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    switch (xdt) {
    case DT_F32: return launch_kernel(k_normalize<DT_F32>, (int)grid, s, x, n, absmax, B, out);
    case DT_F16: return launch_kernel(k_normalize<DT_F16>, (int)grid, s, x, n, absmax, B, out);
    case DT_BF16: return launch_kernel(k_normalize<DT_BF16>, (int)grid, s, x, n, absmax, B, out);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dq_mean(const QuantDesc& single, const TileMap<QuantDesc>* map, int count,
                          const unsigned long long* bins, hipStream_t s)
{
    if (map) return launch_kernel(k_dq_mean<true>, count, s, single, *map, bins);
    return launch_kernel(k_dq_mean<false>, 1, s, single, TileMap<QuantDesc>{}, bins);
}

}  // namespace qb
