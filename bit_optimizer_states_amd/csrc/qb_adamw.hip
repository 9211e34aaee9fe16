// qb_adamw.hip -- fused AdamW step with block-wise dynamic 8-bit moments.
//
// The 8-bit optimizer keeps both Adam moments as block-wise dynamic 8-bit
// codes plus one fp32 absmax per block (abstract quoted on "Py之bitsandbytes：
// bitsandbytes的简介、安装、使用方法之详细攻略", section 2; 2 bytes of state per
// parameter: "bitsandbytes - Quantização de LLM", section Workflow 3) and is a
// drop-in replacement for AdamW (same lr, betas, eps).  One pass per block, in
// registers: decode m and v, update m, v and p, reduce the new block absmax of
// m' and v', encode m' and v' again.  Each parameter's 14-16 bytes cross HBM
// once.
//
// One kernel serves one tensor (descriptor passed by value) or many tensors
// (a descriptor table in device memory; a persistent workgroup walks the
// global tile index upward, so its cursor into the table only moves forward).
#include "qb_device.h"
#include "qb_launch.h"

namespace qb {

template <int B>
struct TileA {
    static constexpr int EPT = B >= 1024 ? B / 256 : 4;
    static constexpr int LPB = B / EPT;
    static constexpr int BPT = kThreads / LPB;
    static constexpr int CH = EPT / 4;
    static constexpr int ELEMS = kThreads * EPT;
    static constexpr int WPB = LPB > 64 ? LPB / 64 : 1;
};

// Block maxima of two non-negative values (as bits), one barrier per tile.
template <class T>
__device__ __forceinline__ void block_max2(uint32_t& x, uint32_t& y, uint32_t (*red)[4], int tid)
{
    constexpr int L = T::LPB < 64 ? T::LPB : 64;
    x = lanes_max<L>(x);
    y = lanes_max<L>(y);
    if constexpr (T::WPB > 1) {
        const int w = tid >> 6;
        if ((tid & 63) == 0) {
            red[0][w] = x;
            red[1][w] = y;
        }
        __syncthreads();
        const int first = (w / T::WPB) * T::WPB;
        uint32_t a = 0, b = 0;
#pragma unroll
        for (int i = 0; i < T::WPB; ++i) {
            a = max(a, red[0][first + i]);
            b = max(b, red[1][first + i]);
        }
        x = a;
        y = b;
    }
}

template <int B, int GDT, bool MULTI>
__global__ __launch_bounds__(256) void k_adamw8(TensorDesc single, const TensorDesc* __restrict__ descs, int count,
                                                int64_t ntiles, AdamScalars hs, const QbTables* __restrict__ tab)
{
    using T = TileA<B>;
    __shared__ float s_dyn[256];
    __shared__ uint2 s_lut[kDynLutN];
    __shared__ uint32_t s_red[2][2][4];
    const int tid = threadIdx.x;
    s_dyn[tid] = tab->dyn8[tid];
    const uint2* glut = reinterpret_cast<const uint2*>(tab->dyn8_lut);
    for (int i = tid; i < kDynLutN; i += kThreads) s_lut[i] = glut[i];
    __syncthreads();

    const int bt = tid / T::LPB, l = tid % T::LPB;
    int cur = 0;
    int par = 0;
    for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x, par ^= 1) {
        TensorDesc d;
        int64_t lt;
        if constexpr (MULTI) {
            while (cur + 1 < count && tile >= descs[cur + 1].tile_begin) ++cur;
            d = descs[cur];
            lt = tile - d.tile_begin;
        } else {
            d = single;
            lt = tile;
        }
        const int64_t nloc = d.n;
        const int64_t nbl = (nloc + B - 1) / B;
        const int64_t blk = lt * T::BPT + bt;
        const int64_t bstart = blk * B;
        const bool full = (lt + 1) * T::ELEMS <= nloc;

        float am0 = 0.0f, av0 = 0.0f;
        if (blk < nbl) {
            am0 = d.am[blk];
            av0 = d.av[blk];
        }
        float p[T::EPT], g[T::EPT];
        uint32_t cmw[T::CH], cvw[T::CH];
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                const int64_t e0 = bstart + c * T::LPB * 4 + l * 4;
                load4<DT_F32>(d.p, e0, &p[c * 4]);
                load4<GDT>(d.g, e0, &g[c * 4]);
                cmw[c] = *reinterpret_cast<const uint32_t*>(d.m + e0);
                cvw[c] = *reinterpret_cast<const uint32_t*>(d.v + e0);
            }
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                uint32_t wm = 0x7F7F7F7Fu, wv = 0x7F7F7F7Fu;   // code of 0.0 in every byte
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                    float pv = 0.0f, gv = 0.0f;
                    if (idx < nloc) {
                        pv = d.p[idx];
                        gv = load1<GDT>(d.g, idx);
                        wm = (wm & ~(0xFFu << (8 * j))) | ((uint32_t)d.m[idx] << (8 * j));
                        wv = (wv & ~(0xFFu << (8 * j))) | ((uint32_t)d.v[idx] << (8 * j));
                    }
                    p[c * 4 + j] = pv;
                    g[c * 4 + j] = gv;
                }
                cmw[c] = wm;
                cvw[c] = wv;
            }
        }

        // decode, update (binary32, every operation rounded on its own)
        float m1[T::EPT], v1[T::EPT];
        uint32_t mxm = 0, mxv = 0;
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const uint32_t sh = 8 * (i & 3);
            const float m0 = s_dyn[(cmw[i >> 2] >> sh) & 0xFFu] * am0;
            const float v0 = s_dyn[(cvw[i >> 2] >> sh) & 0xFFu] * av0;
            const float gi = g[i];
            const float mm = hs.b1 * m0 + hs.ob1 * gi;
            const float vv = hs.b2 * v0 + hs.ob2 * (gi * gi);
            const float den = sqrtf(vv) * hs.s2 + hs.eps;
            p[i] = p[i] * hs.dec - hs.s1 * (mm / den);
            m1[i] = mm;
            v1[i] = vv;
            mxm = max(mxm, fbits(mm) & 0x7FFFFFFFu);
            mxv = max(mxv, fbits(vv) & 0x7FFFFFFFu);
        }
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
                *reinterpret_cast<float4*>(d.p + bstart + c * T::LPB * 4 + l * 4) =
                    make_float4(p[c * 4], p[c * 4 + 1], p[c * 4 + 2], p[c * 4 + 3]);
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                    if (idx < nloc) d.p[idx] = p[c * 4 + j];
                }
        }

        // new block absmax of m' and v'
        block_max2<T>(mxm, mxv, s_red[par], tid);
        const float am1 = ffrom(mxm), av1 = ffrom(mxv);
        if (l == 0 && blk < nbl) {
            d.am[blk] = am1;
            d.av[blk] = av1;
        }

        // encode m' (signed) and v' (non-negative) with the dynamic code
        const float rm = am1 > 0.0f ? 1.0f / am1 : 0.0f;
        const float rv = av1 > 0.0f ? 1.0f / av1 : 0.0f;
        const bool fast = fast_div_ok(am1) && fast_div_ok(av1);
        uint32_t om[T::CH], ov[T::CH];
        if (__all(fast)) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                uint32_t wm = 0, wv = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    wm |= enc_dyn8(div_by_block(m1[c * 4 + j], am1, rm), s_lut) << (8 * j);
                    wv |= enc_dyn8_pos(div_by_block(v1[c * 4 + j], av1, rv), s_lut) << (8 * j);
                }
                om[c] = wm;
                ov[c] = wv;
            }
        } else {
            const bool fm = fast_div_ok(am1), fv = fast_div_ok(av1);
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                uint32_t wm = 0, wv = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float mm = m1[c * 4 + j], vv = v1[c * 4 + j];
                    const float nm = fm ? div_by_block(mm, am1, rm) : (am1 > 0.0f ? mm / am1 : 0.0f);
                    const float nv = fv ? div_by_block(vv, av1, rv) : (av1 > 0.0f ? vv / av1 : 0.0f);
                    wm |= enc_dyn8(nm, s_lut) << (8 * j);
                    wv |= enc_dyn8_pos(nv, s_lut) << (8 * j);
                }
                om[c] = wm;
                ov[c] = wv;
            }
        }
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                const int64_t e0 = bstart + c * T::LPB * 4 + l * 4;
                *reinterpret_cast<uint32_t*>(d.m + e0) = om[c];
                *reinterpret_cast<uint32_t*>(d.v + e0) = ov[c];
            }
        } else {
#pragma unroll
            for (int c = 0; c < T::CH; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t idx = bstart + c * T::LPB * 4 + l * 4 + j;
                    if (idx < nloc) {
                        d.m[idx] = (uint8_t)(om[c] >> (8 * j));
                        d.v[idx] = (uint8_t)(ov[c] >> (8 * j));
                    }
                }
        }
    }
}

int64_t adamw_tiles(int64_t n, int B)
{
    const int64_t elems = (int64_t)kThreads * (B >= 1024 ? B / 256 : 4);
    return (n + elems - 1) / elems;
}

namespace {

template <int B, int GDT>
hipError_t adamw_as(const TensorDesc& single, const TensorDesc* descs, int count, int64_t ntiles,
                    const AdamScalars& hs, const QbTables* tab, hipStream_t s)
{
    static_assert(TileA<B>::ELEMS == kThreads * (B >= 1024 ? B / 256 : 4), "tile size");
    if (descs) {
        auto kern = k_adamw8<B, GDT, true>;
        return launch_kernel(kern, persistent_grid(kern, ntiles), s, single, descs, count, ntiles, hs, tab);
    }
    auto kern = k_adamw8<B, GDT, false>;
    return launch_kernel(kern, persistent_grid(kern, ntiles), s, single, descs, count, ntiles, hs, tab);
}

template <int B>
hipError_t adamw_dt(int gdt, const TensorDesc& single, const TensorDesc* descs, int count, int64_t ntiles,
                    const AdamScalars& hs, const QbTables* tab, hipStream_t s)
{
    switch (gdt) {
    case DT_F32: return adamw_as<B, DT_F32>(single, descs, count, ntiles, hs, tab, s);
    case DT_F16: return adamw_as<B, DT_F16>(single, descs, count, ntiles, hs, tab, s);
    case DT_BF16: return adamw_as<B, DT_BF16>(single, descs, count, ntiles, hs, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_adamw8(const TensorDesc& single, const TensorDesc* descs, int count, int64_t ntiles, int B,
                         int gdt, const AdamScalars& hs, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    switch (B) {
    case 64: return adamw_dt<64>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 128: return adamw_dt<128>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 256: return adamw_dt<256>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 512: return adamw_dt<512>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 1024: return adamw_dt<1024>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 2048: return adamw_dt<2048>(gdt, single, descs, count, ntiles, hs, tab, s);
    case 4096: return adamw_dt<4096>(gdt, single, descs, count, ntiles, hs, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qb
