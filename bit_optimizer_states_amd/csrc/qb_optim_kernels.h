// qb_optim_kernels.h -- the kernels of the fused 8-bit optimizer steps (AdamW,
// Adam, Lion, SGD with momentum, RMSprop and the layer-wise LAMB and LARS,
// each state held as block-wise dynamic 8-bit codes) and their dispatch over
// kind, block size and dtypes.  Shared by qb_optim.hip (every state in the
// signed dynamic code) and qb_optim_uv.hip (the never-negative state in the
// unsigned dynamic code), which instantiate one half each and compile in
// parallel.
//
// The 8-bit optimizer keeps its states as block-wise dynamic 8-bit codes plus
// one fp32 absmax per block (abstract quoted on "Py之bitsandbytes：
// bitsandbytes的简介、安装、使用方法之详细攻略", section 2; 2 bytes of state per
// parameter for Adam: "bitsandbytes - Quantização de LLM", section Workflow
// 3) and replaces its 32-bit optimizer with the same hyperparameters; 8-bit
// Adam, SGD, RMSprop and Lion are listed beside AdamW ("bitsandbytes深度解析",
// section 优化器模块深度分析).  One pass per block, in registers: decode the
// states, update them and p, reduce each state's new block absmax, encode the
// states again.  Each parameter's bytes cross HBM once.
//
// One 256-thread workgroup per tile (a tile is one block for B >= 1024), in
// tile order.  For many tensors, the tiles of all tensors are numbered in one
// range; a workgroup finds its tensor from a coarse bucket index (the tensor
// holding the bucket's first tile) and, only where a bucket spans several
// tensors, a binary search among those (uniform, scalar loads that stay in
// the scalar cache).  Parameters are binary32, or 16-bit (widened on load,
// rounded once to nearest even on store).  The layer-wise kinds LAMB and
// LARS need each tensor's norms before any parameter moves: a norm pass
// (k_trust_norms, k_trust_scalars) precedes their step.
#pragma once
#include "qb_device.h"
#include "qb_launch.h"

namespace qb {

// Threads per workgroup of the optimizer kernel: a 2048-element block takes one
// workgroup of kAdamThreads threads, i.e. 2048 / kAdamThreads elements per
// thread; more elements per thread spread the per-block fixed work (tensor
// lookup, table staging, block reduction, reciprocals) thinner.  Measured on
// MI355X in one process on the 7B step: 128 and 512 threads are 3-5% slower.
#ifndef QB_ADAM_THREADS
#define QB_ADAM_THREADS 256
#endif
constexpr int kAdamThreads = QB_ADAM_THREADS;

// Resident workgroups per CU of the fused step with binary32 parameters, held
// there by reserving LDS at launch (the AdamW step's registers would allow 7,
// the one-state kinds' 8).  Measured on MI355X, same process and buffers,
// results bit-identical: 6 is 0.8-1.6% faster than 7 on the 7B AdamW step
// (four boxes), 1.1-1.4% on AdamW over a flat 1.5e9 buffer and 2-3% on Lion,
// SGD and RMSprop there, Adam within +-1%; 5 and 4 are 2% slower.  The AdamW
// step's memory accesses alone (no arithmetic) show the same optimum: 3%
// faster at 6 than at 8.  With 16-bit parameters (fewer bytes per element)
// the cap measured 1-5% slower, so those launches keep the occupancy their
// resources give.
#ifndef QB_ADAM_WGS_PER_CU
#define QB_ADAM_WGS_PER_CU 6
#endif

// XCD-contiguous tile order (tile_of): measured on MI355X in one process (the
// same buffers), 4-6% faster than the plain order on the 7B step.
#ifndef QB_TILE_REMAP
#define QB_TILE_REMAP 1
#endif

// Elements a thread takes per access: 4 (chunks spread over the block) or 8
// (each thread owns 8 consecutive elements: wider gradient and code accesses).
// Measured on MI355X: 8 is 7-9% slower (flat 1.5e9 parameters and 7B step).
#ifndef QB_ADAM_CHUNK
#define QB_ADAM_CHUNK 4
#endif

template <int B>
struct TileA {
    static constexpr int BS = B;                                         // block size
    static constexpr int NT = kAdamThreads;
    static constexpr int EPT = B >= 4 * NT ? B / NT : 4;
    static constexpr int CW = (QB_ADAM_CHUNK == 8 && EPT % 8 == 0) ? 8 : 4;   // elements per chunk
    static constexpr int LPB = B / EPT;
    static constexpr int BPT = NT / LPB;
    static constexpr int CH = EPT / CW;
    static constexpr int ELEMS = NT * EPT;
    static constexpr int WPB = LPB > 64 ? LPB / 64 : 1;
};

// CW consecutive elements of dtype DT at element offset e.
template <int DT, int CW>
__device__ __forceinline__ void load_chunk(const void* base, uint32_t e, float* v)
{
    if constexpr (CW == 4) load4o<DT>(base, e, v);
    else load8o<DT>(base, e, v);
}

template <int CW>
__device__ __forceinline__ void load_codes(const uint8_t* base, uint32_t e, uint32_t* w)
{
    if constexpr (CW == 4) {
        w[0] = gldo<uint32_t>(base, e);
    } else {
        const u32x2 x = gldo<u32x2>(base, e);
        w[0] = x.x;
        w[1] = x.y;
    }
}

template <int CW>
__device__ __forceinline__ void store_codes(uint8_t* base, uint32_t e, const uint32_t* w)
{
    if constexpr (CW == 4) {
        gsto<uint32_t>(base, e, w[0]);
    } else {
        const u32x2 x = {w[0], w[1]};
        gsto<u32x2>(base, e, x);
    }
}

// Block maxima of two non-negative values (as bits).
template <class T>
__device__ __forceinline__ void block_max2(uint32_t& x, uint32_t& y, uint32_t (*red)[T::NT / 64], int tid)
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

// States of an optimizer kind: two (m, v) for Adam(W) and LAMB, one otherwise.
constexpr int opt_states(int opt) { return (opt == OPT_ADAMW || opt == OPT_ADAM || opt == OPT_LAMB) ? 2 : 1; }

// LAMB's moments and direction: x, y become m', v' (separately rounded, as
// they decide the codes); returns u = r + wd*p with r = s1*m'/(sqrt(v')*s2 +
// eps) from hardware square root and reciprocal.  The norm pass and the step
// both call this, so they see the same u bit for bit.
__device__ __forceinline__ float lamb_dir(const OptScalars& hs, float gi, float p, float& x, float& y)
{
    const float mm = hs.b1 * x + hs.ob1 * gi;
    const float vv = hs.b2 * y + hs.ob2 * (gi * gi);
    const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(vv), hs.s2, hs.eps);
    const float r = hs.s1 * (mm * __builtin_amdgcn_rcpf(den));
    x = mm;
    y = vv;
    return __builtin_fmaf(hs.wd, p, r);
}

// One element of the update, binary32.  x, y: the decoded states (y for the
// two-state kinds), replaced by the updated ones; p updated in place.  The
// states are computed with every operation rounded on its own, exactly as the
// definitions read, because they decide the codes.  Where a state reads p (the
// L2 term of Adam, SGD and RMSprop) p must be exact too, so those kinds and
// Lion update p with separately rounded operations and IEEE square root and
// division: bit-exact.  AdamW's states never read p, so its parameter update
// takes hardware square root and reciprocal (about 1 ulp each) and fused
// multiply-adds: within 1e-6 relative of the separately rounded formula.
template <int OPT>
__device__ __forceinline__ void opt_elem(const OptScalars& hs, float gi, float& p, float& x, float& y)
{
    if constexpr (OPT == OPT_ADAMW) {
        const float mm = hs.b1 * x + hs.ob1 * gi;
        const float vv = hs.b2 * y + hs.ob2 * (gi * gi);
        const float den = __builtin_fmaf(__builtin_amdgcn_sqrtf(vv), hs.s2, hs.eps);
        const float upd = mm * __builtin_amdgcn_rcpf(den);
        p = __builtin_fmaf(-hs.s1, upd, p * hs.dec);
        x = mm;
        y = vv;
    } else if constexpr (OPT == OPT_ADAM) {               // L2-coupled decay
        const float t = hs.wd * p;
        const float gw = gi + t;
        const float mm = hs.b1 * x + hs.ob1 * gw;
        const float vv = hs.b2 * y + hs.ob2 * (gw * gw);
        const float den = __builtin_sqrtf(vv) * hs.s2 + hs.eps;
        p = p - hs.s1 * (mm / den);
        x = mm;
        y = vv;
    } else if constexpr (OPT == OPT_LION) {
        const float c = hs.b1 * x + hs.ob1 * gi;
        const float sg = c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
        p = p * hs.dec - hs.lr * sg;                       // lr * sign is exact
        x = hs.b2 * x + hs.ob2 * gi;
    } else if constexpr (OPT == OPT_SGD) {
        const float t = hs.wd * p;
        const float gw = gi + t;
        const float buf = (hs.flags & kOptFirstStep) ? gw : hs.b1 * x + hs.omd * gw;
        const float dir = (hs.flags & kOptNesterov) ? gw + hs.b1 * buf : buf;
        p = p - hs.lr * dir;
        x = buf;
    } else if constexpr (OPT == OPT_RMSPROP) {
        const float t = hs.wd * p;
        const float gw = gi + t;
        const float vv = hs.b2 * x + hs.ob2 * (gw * gw);
        const float den = __builtin_sqrtf(vv) + hs.eps;
        p = p - hs.lr * (gw / den);
        x = vv;
    } else if constexpr (OPT == OPT_LAMB) {               // hs.lr = the tensor's S
        const float u = lamb_dir(hs, gi, p, x, y);
        p = __builtin_fmaf(-hs.lr, u, p);
    } else {                                               // LARS; hs.lr = the tensor's S
        const float t = hs.wd * p;
        const float gw = gi + t;
        const float buf = hs.b1 * x + hs.lr * gw;
        p = p - buf;
        x = buf;
    }
}

// A tile of a tensor whose states stay binary32 (the 32-bit fallback for small
// or chosen tensors: d.am == nullptr, d.m / d.v are float arrays).  The same
// element update, with no codes and no block absmax.
template <int OPT, class T, int GDT, int PDT>
__device__ __forceinline__ void optim32_tile(const TensorDesc& d, int64_t lt, const OptScalars& hs, int tid)
{
    constexpr bool TWO = opt_states(OPT) == 2;
    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t tbase = lt * T::ELEMS;
    void* const pt = static_cast<char*>(d.p) + tbase * (PDT == DT_F32 ? 4 : 2);
    const void* const gt = static_cast<const char*>(d.g) + tbase * (GDT == DT_F32 ? 4 : 2);
    float* const xt = reinterpret_cast<float*>(d.m) + tbase;
    float* const yt = TWO ? reinterpret_cast<float*>(d.v) + tbase : nullptr;
    const uint32_t lofs = (uint32_t)(bt * T::BS + l * T::CW);
    const int64_t lrem = d.n - tbase;
    const bool full = T::ELEMS <= lrem;
    float p[T::EPT], g[T::EPT], x[T::EPT], y[T::EPT];
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            const uint32_t e = lofs + c * T::LPB * T::CW;
            load_chunk<PDT, T::CW>(pt, e, &p[c * T::CW]);
            load_chunk<GDT, T::CW>(gt, e, &g[c * T::CW]);
            load_chunk<DT_F32, T::CW>(xt, e, &x[c * T::CW]);
            if constexpr (TWO) load_chunk<DT_F32, T::CW>(yt, e, &y[c * T::CW]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
            const bool in = (int64_t)e < lrem;
            p[i] = in ? load1<PDT>(pt, e) : 0.0f;
            g[i] = in ? load1<GDT>(gt, e) : 0.0f;
            x[i] = in ? load1<DT_F32>(xt, e) : 0.0f;
            y[i] = (TWO && in) ? load1<DT_F32>(yt, e) : 0.0f;
        }
    }
#pragma unroll
    for (int i = 0; i < T::EPT; ++i) opt_elem<OPT>(hs, g[i], p[i], x[i], y[i]);
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c)
#pragma unroll
            for (int h = 0; h < T::CW; h += 4) {
                const uint32_t e = lofs + c * T::LPB * T::CW + h;
                store4o<PDT>(pt, e, &p[c * T::CW + h]);
                store4o<DT_F32>(xt, e, &x[c * T::CW + h]);
                if constexpr (TWO) store4o<DT_F32>(yt, e, &y[c * T::CW + h]);
            }
    } else {
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
            if ((int64_t)e < lrem) {
                store1o<PDT>(pt, e, p[i]);
                gsto<float>(xt, e * 4u, x[i]);
                if constexpr (TWO) gsto<float>(yt, e * 4u, y[i]);
            }
        }
    }
}

// Where the never-negative state (v of the two-state kinds, the state of
// RMSprop) is held in the unsigned dynamic code, UV is true: its decode and
// encode tables are staged beside the signed ones, and its code of 0.0 is 0.
template <bool UV>
struct VCodeLds {
    float dec[256];
    UDynEncLds enc;
};
template <>
struct VCodeLds<false> {
    float dec[1];
};

template <int OPT, int B, int GDT, bool MULTI, int PDT, bool UV>
__global__ __launch_bounds__(kAdamThreads) void k_optim8(TensorDesc single, TileMap<TensorDesc> map, OptScalars hs0,
                                                         const QbTables* __restrict__ tab,
                                                         const float* __restrict__ trust)
{
    using T = TileA<B>;
    constexpr bool TWO = opt_states(OPT) == 2;
    constexpr bool X_POS = OPT == OPT_RMSPROP;             // the one state of RMSprop is >= 0
    static_assert(!UV || TWO || X_POS, "the unsigned code needs a never-negative state");
    constexpr bool SIGNED = !(UV && X_POS);                // some state uses the signed code
    constexpr uint32_t kZeroX = SIGNED ? 0x7F7F7F7Fu : 0u;  // code of 0.0 in every byte
    constexpr uint32_t kZeroY = UV ? 0u : 0x7F7F7F7Fu;
    __shared__ float s_dyn[SIGNED ? 256 : 1];
    __shared__ DynEncLds s_enc;
    __shared__ VCodeLds<UV> s_v;
    __shared__ uint32_t s_red[2][T::NT / 64];
    const int tid = threadIdx.x;
    const int64_t tile = tile_of<QB_TILE_REMAP>(blockIdx.x, gridDim.x);

    TensorDesc d;
    int64_t lt;
    OptScalars hs = hs0;
    if constexpr (MULTI) {
        const int ti = find_tensor(map, tile);
        d = map.descs[ti];
        lt = tile - d.tile_begin;
        if constexpr (opt_layerwise(OPT)) hs.lr = trust[ti];
    } else {
        d = single;
        lt = tile;
    }
    if (d.am == nullptr) {                                 // binary32 states (uniform per workgroup)
        optim32_tile<OPT, T, GDT, PDT>(d, lt, hs, tid);
        return;
    }
    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nloc = d.n;
    const int64_t nbl = (nloc + B - 1) / B;
    const int64_t blk = lt * T::BPT + bt;
    const bool full = (lt + 1) * T::ELEMS <= nloc;
    // uniform tile base pointers; per-lane offsets stay 32-bit
    const int64_t tbase = lt * T::ELEMS;
    void* const pt = static_cast<char*>(d.p) + tbase * (PDT == DT_F32 ? 4 : 2);
    const void* const gt = static_cast<const char*>(d.g) + tbase * (GDT == DT_F32 ? 4 : 2);
    uint8_t* const mt = d.m + tbase;
    uint8_t* const vt = TWO ? d.v + tbase : nullptr;
    const uint32_t lofs = (uint32_t)(bt * B + l * T::CW);  // element offset of chunk 0 in the tile
    const int64_t lrem = nloc - tbase;                      // elements left in the tensor from the tile start

    // loads first; the tables are staged while they are in flight
    float am0 = 0.0f, av0 = 0.0f;
    if (blk < nbl) {
        am0 = gld<float>(d.am + blk);
        if constexpr (TWO) av0 = gld<float>(d.av + blk);
    }
    float p[T::EPT], g[T::EPT];
    uint32_t cmw[T::EPT / 4], cvw[T::EPT / 4];             // 4 codes per word
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            const uint32_t e = lofs + c * T::LPB * T::CW;
            load_chunk<PDT, T::CW>(pt, e, &p[c * T::CW]);
            load_chunk<GDT, T::CW>(gt, e, &g[c * T::CW]);
            load_codes<T::CW>(mt, e, &cmw[c * T::CW / 4]);
            if constexpr (TWO) load_codes<T::CW>(vt, e, &cvw[c * T::CW / 4]);
        }
    } else {
#pragma unroll
        for (int w = 0; w < T::EPT / 4; ++w) {
            uint32_t wm = kZeroX, wv = kZeroY;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = w * 4 + j;                     // element slot: chunk i / CW, lane part i % CW
                const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
                float pv = 0.0f, gv = 0.0f;
                if ((int64_t)e < lrem) {
                    pv = load1<PDT>(pt, e);
                    gv = load1<GDT>(gt, e);
                    wm = (wm & ~(0xFFu << (8 * j))) | ((uint32_t)gldo<uint8_t>(mt, e) << (8 * j));
                    if constexpr (TWO) wv = (wv & ~(0xFFu << (8 * j))) | ((uint32_t)gldo<uint8_t>(vt, e) << (8 * j));
                }
                p[i] = pv;
                g[i] = gv;
            }
            cmw[w] = wm;
            cvw[w] = wv;
        }
    }
    // the code tables: every word is loaded before any is stored (one wait)
    constexpr int kBaseW = kDynBucketBytes / 4;           // one sign's buckets
    StageWords<T::NT, 256> st_dec, st_thr, st_udec, st_uthr;
    StageWords<T::NT, kBaseW> st_pos, st_neg;
    StageWords<T::NT, kUDynBucketBytes / 4> st_ubase;
    if constexpr (SIGNED) {
        st_dec.load(tab->dyn8, tid);
        st_pos.load(&tab->dyn8_base[0][0], tid);
        st_neg.load(&tab->dyn8_base[1][0], tid);
        st_thr.load(tab->dyn8_thr, tid);
    }
    if constexpr (UV) {
        st_udec.load(tab->udyn8, tid);
        st_ubase.load(tab->udyn8_base, tid);
        st_uthr.load(tab->udyn8_thr, tid);
    }
    if constexpr (SIGNED) {
        st_dec.hold();
        st_pos.hold();
        st_neg.hold();
        st_thr.hold();
    }
    if constexpr (UV) {
        st_udec.hold();
        st_ubase.hold();
        st_uthr.hold();
    }
    if constexpr (SIGNED) {
        st_dec.store(s_dyn, tid);
        st_pos.store(&s_enc.base[kDynBase / 4], tid);
        st_neg.store(&s_enc.base[(kDynIdxSign + kDynBase) / 4], tid);
        st_thr.store(s_enc.thr, tid);
    }
    if constexpr (UV) {
        st_udec.store(s_v.dec, tid);
        st_ubase.store(s_v.enc.base, tid);
        st_uthr.store(s_v.enc.thr, tid);
    }
    __syncthreads();
    const float* const dec_x = SIGNED ? s_dyn : s_v.dec;
    const float* const dec_y = UV ? s_v.dec : s_dyn;

    // decode, update
    float m1[T::EPT], v1[T::EPT];
    float mxm = 0.0f, mxv = 0.0f;
#pragma unroll
    for (int i = 0; i < T::EPT; ++i) {
        const uint32_t sh = 8 * (i & 3);
        float x = dec_x[(cmw[i >> 2] >> sh) & 0xFFu] * am0;
        float y = TWO ? dec_y[(cvw[i >> 2] >> sh) & 0xFFu] * av0 : 0.0f;
        opt_elem<OPT>(hs, g[i], p[i], x, y);
        m1[i] = x;
        v1[i] = y;
        mxm = __builtin_fmaxf(mxm, __builtin_fabsf(x));
        if constexpr (TWO) mxv = __builtin_fmaxf(mxv, y);  // v' >= 0
    }
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            store4o<PDT>(pt, lofs + c * T::LPB * T::CW, &p[c * T::CW]);
            if constexpr (T::CW == 8) store4o<PDT>(pt, lofs + c * T::LPB * T::CW + 4, &p[c * T::CW + 4]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
            if ((int64_t)e < lrem) store1o<PDT>(pt, e, p[i]);
        }
    }

    // new block absmax of the states (non-negative floats compare as their bits)
    uint32_t bm = fbits(mxm), bv = fbits(mxv);
    block_max2<T>(bm, bv, s_red, tid);
    const float am1 = ffrom(bm), av1 = ffrom(bv);
    if (l == 0 && blk < nbl) {
        gst<float>(d.am + blk, am1);
        if constexpr (TWO) gst<float>(d.av + blk, av1);
    }

    // encode the states (m' signed; v' >= 0, in the unsigned code where UV)
    const float rm = rcp_rn(am1);        // used only where fast_div_ok(am1)
    const float rv = rcp_rn(av1);
    const bool fm = fast_div_ok(am1), fv = !TWO || fast_div_ok(av1);
    uint32_t om[T::EPT / 4], ov[T::EPT / 4];
    auto enc_x = [&](float nv) -> uint32_t {
        if constexpr (!SIGNED) return enc_udyn8(nv, s_v.enc);
        else return X_POS ? enc_dyn8_pos(nv, s_enc) : enc_dyn8(nv, s_enc);
    };
    auto enc_y = [&](float nv) -> uint32_t {
        if constexpr (UV) return enc_udyn8(nv, s_v.enc);
        else return enc_dyn8_pos(nv, s_enc);
    };
    if (__all(fm && fv)) {
#pragma unroll
        for (int c = 0; c < T::EPT / 4; ++c) {
            uint32_t wm = 0, wv = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wm |= enc_x(div_by_block(m1[c * 4 + j], am1, rm)) << (8 * j);
                if constexpr (TWO) wv |= enc_y(div_by_block(v1[c * 4 + j], av1, rv)) << (8 * j);
            }
            om[c] = wm;
            ov[c] = wv;
        }
    } else {
#pragma unroll
        for (int c = 0; c < T::EPT / 4; ++c) {
            uint32_t wm = 0, wv = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float mm = m1[c * 4 + j];
                const float nm = normalize_by_block(mm, am1, rm, fm);
                wm |= enc_x(nm) << (8 * j);
                if constexpr (TWO) {
                    const float vv = v1[c * 4 + j];
                    const float nv = normalize_by_block(vv, av1, rv, fv);
                    wv |= enc_y(nv) << (8 * j);
                }
            }
            om[c] = wm;
            ov[c] = wv;
        }
    }
    if (full) {
#pragma unroll
        for (int c = 0; c < T::CH; ++c) {
            const uint32_t e = lofs + c * T::LPB * T::CW;
            store_codes<T::CW>(mt, e, &om[c * T::CW / 4]);
            if constexpr (TWO) store_codes<T::CW>(vt, e, &ov[c * T::CW / 4]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
            if ((int64_t)e < lrem) {
                gsto<uint8_t>(mt, e, (uint8_t)(om[i >> 2] >> (8 * (i & 3))));
                if constexpr (TWO) gsto<uint8_t>(vt, e, (uint8_t)(ov[i >> 2] >> (8 * (i & 3))));
            }
        }
    }
}

// Layer-wise kinds, first pass: one workgroup per group of kNormGroupTiles
// consecutive optimizer tiles of one tensor (the tiles of k_optim8) adds |p|^2
// and |u|^2 (LAMB: u from the decoded states, as the step will compute it) or
// |g|^2 (LARS) in binary64: each thread over its own elements, tile after
// tile, then across the wave (butterfly) and the waves (in order).  The same
// bits on every run.
template <int OPT, int B, int GDT, int PDT, bool UV>
__global__ __launch_bounds__(kAdamThreads) void k_trust_norms(TileMap<TensorDesc> gmap, OptScalars hs,
                                                              const QbTables* __restrict__ tab,
                                                              double* __restrict__ part)
{
    using T = TileA<B>;
    constexpr bool LAMB = OPT == OPT_LAMB;
    static_assert(!UV || LAMB, "the unsigned code needs a never-negative state");
    __shared__ float s_dyn[256];
    __shared__ float s_udyn[UV ? 256 : 1];
    __shared__ double s_red[2][T::NT / 64];
    const int tid = threadIdx.x;
    const int64_t grp = tile_of<QB_TILE_REMAP>(blockIdx.x, gridDim.x);
    const TensorDesc d = gmap.descs[find_tensor(gmap, grp)];
    const int64_t tiles = (d.n + T::ELEMS - 1) / T::ELEMS;
    const int64_t lt0 = (grp - d.tile_begin) * kNormGroupTiles;
    const int64_t lt1 = lt0 + kNormGroupTiles < tiles ? lt0 + kNormGroupTiles : tiles;
    const int bt = tid / T::LPB, l = tid % T::LPB;
    const int64_t nbl = (d.n + B - 1) / B;
    const bool s8 = d.am != nullptr;                       // uniform per workgroup
    const uint32_t lofs = (uint32_t)(bt * B + l * T::CW);
    if (LAMB && s8) {
#pragma unroll
        for (int r = 0; r < (256 + T::NT - 1) / T::NT; ++r)
            if (T::NT <= 256 || tid < 256) s_dyn[r * T::NT + tid] = tab->dyn8[r * T::NT + tid];
        if constexpr (UV) {
#pragma unroll
            for (int r = 0; r < (256 + T::NT - 1) / T::NT; ++r)
                if (T::NT <= 256 || tid < 256) s_udyn[r * T::NT + tid] = tab->udyn8[r * T::NT + tid];
        }
        __syncthreads();
    }
    const float* const dec_v = UV ? s_udyn : s_dyn;
    double sp = 0.0, sq = 0.0;
    for (int64_t lt = lt0; lt < lt1; ++lt) {
        const int64_t blk = lt * T::BPT + bt;
        const int64_t tbase = lt * T::ELEMS;
        const int64_t lrem = d.n - tbase;
        const bool full = T::ELEMS <= lrem;
        const void* const pt = static_cast<const char*>(d.p) + tbase * (PDT == DT_F32 ? 4 : 2);
        const void* const gt = static_cast<const char*>(d.g) + tbase * (GDT == DT_F32 ? 4 : 2);
        float am0 = 0.0f, av0 = 0.0f;
        if (LAMB && s8 && blk < nbl) {
            am0 = gld<float>(d.am + blk);
            av0 = gld<float>(d.av + blk);
        }
        // elements past the end read as p = g = 0 and state 0: they add exactly 0
        float p[T::EPT], g[T::EPT], x[T::EPT], y[T::EPT];
        uint32_t cmw[T::EPT / 4], cvw[T::EPT / 4];
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) x[i] = y[i] = 0.0f;
#pragma unroll
        for (int w = 0; w < T::EPT / 4; ++w) {
            cmw[w] = 0x7F7F7F7Fu;                          // codes of 0.0
            cvw[w] = UV ? 0u : 0x7F7F7F7Fu;
        }
        if (full) {
#pragma unroll
            for (int c = 0; c < T::CH; ++c) {
                const uint32_t e = lofs + c * T::LPB * T::CW;
                load_chunk<PDT, T::CW>(pt, e, &p[c * T::CW]);
                load_chunk<GDT, T::CW>(gt, e, &g[c * T::CW]);
                if constexpr (LAMB) {
                    if (s8) {
                        load_codes<T::CW>(d.m + tbase, e, &cmw[c * T::CW / 4]);
                        load_codes<T::CW>(d.v + tbase, e, &cvw[c * T::CW / 4]);
                    } else {
                        load_chunk<DT_F32, T::CW>(reinterpret_cast<float*>(d.m) + tbase, e, &x[c * T::CW]);
                        load_chunk<DT_F32, T::CW>(reinterpret_cast<float*>(d.v) + tbase, e, &y[c * T::CW]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < T::EPT; ++i) {
                const uint32_t e = lofs + (i / T::CW) * T::LPB * T::CW + (i % T::CW);
                const bool in = (int64_t)e < lrem;
                p[i] = in ? load1<PDT>(pt, e) : 0.0f;
                g[i] = in ? load1<GDT>(gt, e) : 0.0f;
                if constexpr (LAMB) {
                    if (in && s8) {
                        const uint32_t sh = 8 * (i & 3), keep = ~(0xFFu << sh);
                        cmw[i >> 2] = (cmw[i >> 2] & keep) | ((uint32_t)gldo<uint8_t>(d.m + tbase, e) << sh);
                        cvw[i >> 2] = (cvw[i >> 2] & keep) | ((uint32_t)gldo<uint8_t>(d.v + tbase, e) << sh);
                    } else if (in) {
                        x[i] = load1<DT_F32>(reinterpret_cast<float*>(d.m) + tbase, e);
                        y[i] = load1<DT_F32>(reinterpret_cast<float*>(d.v) + tbase, e);
                    }
                }
            }
        }
        if (LAMB && s8) {
#pragma unroll
            for (int i = 0; i < T::EPT; ++i) {
                const uint32_t sh = 8 * (i & 3);
                x[i] = s_dyn[(cmw[i >> 2] >> sh) & 0xFFu] * am0;
                y[i] = dec_v[(cvw[i >> 2] >> sh) & 0xFFu] * av0;
            }
        }
#pragma unroll
        for (int i = 0; i < T::EPT; ++i) {
            const double pd = (double)p[i];
            sp = __builtin_fma(pd, pd, sp);                // the square is exact in binary64
            if constexpr (LAMB) {
                const double u = (double)lamb_dir(hs, g[i], p[i], x[i], y[i]);
                sq = __builtin_fma(u, u, sq);
            } else {
                const double gd = (double)g[i];
                sq = __builtin_fma(gd, gd, sq);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        sp += __shfl_xor(sp, off);
        sq += __shfl_xor(sq, off);
    }
    if ((tid & 63) == 0) {
        s_red[0][tid >> 6] = sp;
        s_red[1][tid >> 6] = sq;
    }
    __syncthreads();
    if (tid == 0) {
        double a = 0.0, b = 0.0;
#pragma unroll
        for (int w = 0; w < T::NT / 64; ++w) {
            a += s_red[0][w];
            b += s_red[1][w];
        }
        part[2 * grp] = a;
        part[2 * grp + 1] = b;
    }
}


namespace optim_dispatch {

// Launch arguments shared by the optimizer launches.
struct OptLaunch {
    const TensorDesc* single;
    const TileMap<TensorDesc>* map;
    int64_t ntiles;
    const OptScalars* hs;
    const QbTables* tab;
    const float* trust;      // k_optim8 of the layer-wise kinds
    double* part;            // non-null: launch k_trust_norms instead
    int pdt;                 // parameter dtype
    hipStream_t s;
};

template <int OPT, int B, int GDT, int PDT, bool UV>
hipError_t optim_as(const OptLaunch& a)
{
    static_assert(TileA<B>::ELEMS == kAdamThreads * (B >= 4 * kAdamThreads ? B / kAdamThreads : 4), "tile size");
    if (a.ntiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    constexpr int kWgs = PDT == DT_F32 ? QB_ADAM_WGS_PER_CU : 0;   // 0: no cap
    auto lds = [](auto kern) { return kWgs ? lds_for_wgs_per_cu(reinterpret_cast<const void*>(kern), kWgs) : 0; };
    if constexpr (opt_layerwise(OPT)) {                   // multi-tensor only (the norms need a workspace)
        if (!a.map) return hipErrorInvalidValue;
        if (a.part)
            return launch_kernel_nt(k_trust_norms<OPT, B, GDT, PDT, UV>, (int)a.ntiles, kAdamThreads, a.s, *a.map, *a.hs,
                                    a.tab, a.part);
        constexpr auto kern = k_optim8<OPT, B, GDT, true, PDT, UV>;
        return launch_kernel_lds(kern, (int)a.ntiles, kAdamThreads, lds(kern), a.s, *a.single, *a.map, *a.hs, a.tab,
                                 a.trust);
    } else {
        if (a.map) {
            constexpr auto kern = k_optim8<OPT, B, GDT, true, PDT, UV>;
            return launch_kernel_lds(kern, (int)a.ntiles, kAdamThreads, lds(kern), a.s, *a.single, *a.map, *a.hs,
                                     a.tab, (const float*)nullptr);
        }
        constexpr auto kern = k_optim8<OPT, B, GDT, false, PDT, UV>;
        return launch_kernel_lds(kern, (int)a.ntiles, kAdamThreads, lds(kern), a.s, *a.single, TileMap<TensorDesc>{},
                                 *a.hs, a.tab, (const float*)nullptr);
    }
}

// (parameter, gradient) dtypes: binary32 parameters with any gradient dtype,
// or 16-bit parameters with gradients of the same type.
template <int OPT, int B, bool UV>
hipError_t optim_dt(int gdt, const OptLaunch& a)
{
    if (a.pdt == DT_F32) {
        switch (gdt) {
        case DT_F32: return optim_as<OPT, B, DT_F32, DT_F32, UV>(a);
        case DT_F16: return optim_as<OPT, B, DT_F16, DT_F32, UV>(a);
        case DT_BF16: return optim_as<OPT, B, DT_BF16, DT_F32, UV>(a);
        default: return hipErrorInvalidValue;
        }
    }
    if (a.pdt != gdt) return hipErrorInvalidValue;
    switch (gdt) {
    case DT_F16: return optim_as<OPT, B, DT_F16, DT_F16, UV>(a);
    case DT_BF16: return optim_as<OPT, B, DT_BF16, DT_BF16, UV>(a);
    default: return hipErrorInvalidValue;
    }
}

template <int OPT, bool UV>
hipError_t optim_b(int B, int gdt, const OptLaunch& a)
{
    switch (B) {
    case 64: return optim_dt<OPT, 64, UV>(gdt, a);
    case 128: return optim_dt<OPT, 128, UV>(gdt, a);
    case 256: return optim_dt<OPT, 256, UV>(gdt, a);
    case 512: return optim_dt<OPT, 512, UV>(gdt, a);
    case 1024: return optim_dt<OPT, 1024, UV>(gdt, a);
    case 2048: return optim_dt<OPT, 2048, UV>(gdt, a);
    case 4096: return optim_dt<OPT, 4096, UV>(gdt, a);
    default: return hipErrorInvalidValue;
    }
}

// UV true: only the kinds with a never-negative state (their other kinds are
// rejected before any launch).
template <bool UV>
hipError_t optim_kind(int opt, int B, int gdt, const OptLaunch& a)
{
    switch (opt) {
    case OPT_ADAMW: return optim_b<OPT_ADAMW, UV>(B, gdt, a);
    case OPT_ADAM: return optim_b<OPT_ADAM, UV>(B, gdt, a);
    case OPT_RMSPROP: return optim_b<OPT_RMSPROP, UV>(B, gdt, a);
    case OPT_LAMB: return optim_b<OPT_LAMB, UV>(B, gdt, a);
    default: break;
    }
    if constexpr (!UV) {
        switch (opt) {
        case OPT_LION: return optim_b<OPT_LION, false>(B, gdt, a);
        case OPT_SGD: return optim_b<OPT_SGD, false>(B, gdt, a);
        case OPT_LARS: return optim_b<OPT_LARS, false>(B, gdt, a);
        default: break;
        }
    }
    return hipErrorInvalidValue;
}

// The instantiations with UV true live in qb_optim_uv.hip.
hipError_t optim_kind_uv(int opt, int B, int gdt, const OptLaunch& a);

}  // namespace optim_dispatch

}  // namespace qb
