// qb_device.h -- device helpers shared by the libqb kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qb_launch.h"
#include "qb_tables.h"

namespace qb {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int kThreads = 256;   // every kernel runs 256-thread workgroups (4 waves)

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float ffrom(uint32_t u) { return __uint_as_float(u); }

// ---------------------------------------------------------------------------
// global-memory access
// ---------------------------------------------------------------------------
//
// Pointers read from memory (the multi-tensor descriptor table) are generic;
// casting to the global address space makes every access a GLOBAL
// instruction instead of FLAT (which also counts against the LDS counter).

#define QB_G __attribute__((address_space(1)))
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ T gld(const void* p)
{
    return *(const QB_G T*)p;
}

template <class T>
__device__ __forceinline__ void gst(void* p, T v)
{
    *(QB_G T*)p = v;
}

// Access at a uniform base pointer plus a 32-bit byte offset: the form the
// GLOBAL instructions take directly (scalar base, vector offset), with no
// 64-bit address arithmetic per lane.
// Streaming data (read once, written once) takes non-temporal loads and
// stores: measured on MI355X, the fused AdamW step runs about 10% faster than
// with ordinary accesses (the same bytes reach HBM either way).
#ifndef QB_NT_LOADS
#define QB_NT_LOADS 1
#endif
#ifndef QB_NT_STORES
#define QB_NT_STORES 1
#endif

template <class T>
__device__ __forceinline__ T gldo(const void* base, uint32_t byte_off)
{
    const QB_G T* p = (const QB_G T*)(static_cast<const char*>(base) + byte_off);
    if constexpr (QB_NT_LOADS) return __builtin_nontemporal_load(p);
    else return *p;
}

template <class T>
__device__ __forceinline__ void gsto(void* base, uint32_t byte_off, T v)
{
    QB_G T* p = (QB_G T*)(static_cast<char*>(base) + byte_off);
    if constexpr (QB_NT_STORES) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// element loads / stores (16-bit types travel as raw halves)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return ffrom(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return ffrom(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w)
{
    _Float16 h;
    uint16_t u = (uint16_t)w;
    __builtin_memcpy(&h, &u, 2);
    return (float)h;
}
__device__ __forceinline__ float f16_hi(uint32_t w) { return f16_lo(w >> 16); }

template <int DT>
__device__ __forceinline__ float half_lo(uint32_t w) { return DT == DT_BF16 ? bf16_lo(w) : f16_lo(w); }
template <int DT>
__device__ __forceinline__ float half_hi(uint32_t w) { return DT == DT_BF16 ? bf16_hi(w) : f16_hi(w); }

// 4 consecutive elements at element index i (16-byte aligned for fp32, 8 for 16-bit).
template <int DT>
__device__ __forceinline__ void load4(const void* base, int64_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        f32x4 x = gld<f32x4>(static_cast<const float*>(base) + i);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        u32x2 x = gld<u32x2>(static_cast<const uint16_t*>(base) + i);
        v[0] = half_lo<DT>(x.x); v[1] = half_hi<DT>(x.x); v[2] = half_lo<DT>(x.y); v[3] = half_hi<DT>(x.y);
    }
}

// 4 consecutive elements at element offset i (uint32) from a uniform base.
template <int DT>
__device__ __forceinline__ void load4o(const void* base, uint32_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        f32x4 x = gldo<f32x4>(base, i * 4u);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        u32x2 x = gldo<u32x2>(base, i * 2u);
        v[0] = half_lo<DT>(x.x); v[1] = half_hi<DT>(x.x); v[2] = half_lo<DT>(x.y); v[3] = half_hi<DT>(x.y);
    }
}

// 8 consecutive elements at element index i (16-byte aligned for every type).
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        load4<DT_F32>(base, i, v);
        load4<DT_F32>(base, i + 4, v + 4);
    } else {
        u32x4 x = gld<u32x4>(static_cast<const uint16_t*>(base) + i);
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = half_lo<DT>(w[k]);
            v[2 * k + 1] = half_hi<DT>(w[k]);
        }
    }
}

// 8 consecutive elements at element offset i (uint32) from a uniform base.
template <int DT>
__device__ __forceinline__ void load8o(const void* base, uint32_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        load4o<DT_F32>(base, i, v);
        load4o<DT_F32>(base, i + 4u, v + 4);
    } else {
        u32x4 x = gldo<u32x4>(base, i * 2u);
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = half_lo<DT>(w[k]);
            v[2 * k + 1] = half_hi<DT>(w[k]);
        }
    }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t i)
{
    if constexpr (DT == DT_F32) {
        return gld<float>(static_cast<const float*>(base) + i);
    } else {
        return half_lo<DT>(gld<uint16_t>(static_cast<const uint16_t*>(base) + i));
    }
}

// binary32 -> 16-bit, round to nearest even (v_cvt_pk_bf16_f32 / v_cvt_f16_f32)
template <int DT>
__device__ __forceinline__ uint32_t to_half_bits(float f)
{
    if constexpr (DT == DT_BF16) {
        __bf16 h = (__bf16)f;
        uint16_t u;
        __builtin_memcpy(&u, &h, 2);
        return u;
    } else {
        // The value must be a rounded binary32 before this conversion: left
        // alone, the compiler folds a preceding binary32 multiply and this
        // conversion into v_fma_mixlo_f16, which rounds once instead of twice.
        // The empty asm (no instruction) hides the multiply from that fold.
        asm("" : "+v"(f));
        _Float16 h = (_Float16)f;
        uint16_t u;
        __builtin_memcpy(&u, &h, 2);
        return u;
    }
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    return to_half_bits<DT>(a) | (to_half_bits<DT>(b) << 16);
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t i, float v)
{
    if constexpr (DT == DT_F32)
        gst<float>(static_cast<float*>(base) + i, v);
    else
        gst<uint16_t>(static_cast<uint16_t*>(base) + i, (uint16_t)to_half_bits<DT>(v));
}

// One output at element offset i (uint32) from a uniform base.
template <int DT>
__device__ __forceinline__ void store1o(void* base, uint32_t i, float v)
{
    if constexpr (DT == DT_F32)
        gsto<float>(base, i * 4u, v);
    else
        gsto<uint16_t>(base, i * 2u, (uint16_t)to_half_bits<DT>(v));
}

// 4 consecutive outputs at element index i.
template <int DT>
__device__ __forceinline__ void store4(void* y, int64_t i, const float* o)
{
    if constexpr (DT == DT_F32) {
        f32x4 v = {o[0], o[1], o[2], o[3]};
        gst<f32x4>(static_cast<float*>(y) + i, v);
    } else {
        u32x2 v = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
        gst<u32x2>(static_cast<uint16_t*>(y) + i, v);
    }
}

// 4 consecutive outputs at element offset i (uint32) from a uniform base.
template <int DT>
__device__ __forceinline__ void store4o(void* y, uint32_t i, const float* o)
{
    if constexpr (DT == DT_F32) {
        f32x4 v = {o[0], o[1], o[2], o[3]};
        gsto<f32x4>(y, i * 4u, v);
    } else {
        u32x2 v = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3])};
        gsto<u32x2>(y, i * 2u, v);
    }
}

// 8 consecutive outputs at element offset i (uint32) from a uniform base.
template <int DT>
__device__ __forceinline__ void store8o(void* y, uint32_t i, const float* o)
{
    if constexpr (DT == DT_F32) {
        store4o<DT_F32>(y, i, o);
        store4o<DT_F32>(y, i + 4u, o + 4);
    } else {
        u32x4 v = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3]), pack2<DT>(o[4], o[5]), pack2<DT>(o[6], o[7])};
        gsto<u32x4>(y, i * 2u, v);
    }
}

// 8 consecutive outputs at element index i.
template <int DT>
__device__ __forceinline__ void store8(void* y, int64_t i, const float* o)
{
    if constexpr (DT == DT_F32) {
        store4<DT_F32>(y, i, o);
        store4<DT_F32>(y, i + 4, o + 4);
    } else {
        u32x4 v = {pack2<DT>(o[0], o[1]), pack2<DT>(o[2], o[3]), pack2<DT>(o[4], o[5]), pack2<DT>(o[6], o[7])};
        gst<u32x4>(static_cast<uint16_t*>(y) + i, v);
    }
}

// ---------------------------------------------------------------------------
// multi-tensor launches
// ---------------------------------------------------------------------------

// Tile handled by workgroup b of ntiles.  The hardware deals workgroups
// round-robin to the 8 XCDs (b % 8); with REMAP each XCD takes one contiguous
// range of tiles instead of every eighth tile (a bijection of [0, ntiles):
// XCD x holds q + (x < r) workgroups, q = ntiles / 8, r = ntiles % 8).  Each
// XCD then streams through one region of every array.  Runs of 16 to 1024
// tiles dealt round-robin measured no better on MI355X.
template <bool REMAP>
__device__ __forceinline__ int64_t tile_of(int64_t b, int64_t ntiles)
{
    if constexpr (REMAP) {
        constexpr int X = 8;
        const int64_t q = ntiles / X, r = ntiles % X;
        const int64_t x = b % X, k = b / X;
        return x * q + (x < r ? x : r) + k;
    } else {
        return b;
    }
}

// Index of the tensor holding global tile `tile`: between the tensor holding
// the first tile of tile's bucket and the one holding the next bucket's first
// tile (usually the same or adjacent ones), by binary search on tile_begin
// (tile_begin[lo] <= tile < tile_begin[hi]).  Uniform: scalar loads.
template <class Desc>
__device__ __forceinline__ int find_tensor(const TileMap<Desc>& map, int64_t tile)
{
    const int64_t k = tile >> map.shift;
    int lo = map.bucket_first[k], hi = map.bucket_first[k + 1] + 1;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (map.tile_begin[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// reductions (non-negative binary32 values compared as unsigned bit patterns)
// ---------------------------------------------------------------------------

// Max over aligned groups of L lanes (L a power of two, <= 64); every lane of
// the group gets the result.  All 64 lanes must be active.
template <int L>
__device__ __forceinline__ uint32_t lanes_max(uint32_t x)
{
    if constexpr (L >= 2) x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    if constexpr (L >= 4) x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    if constexpr (L >= 8) x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));  // row_half_mirror
    if constexpr (L >= 16) x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false)); // row_mirror
    if constexpr (L == 32) {
        // rows are 16 lanes: the maxima of rows 0|1 and 2|3, taken from one
        // lane of each row (uniform scalar values)
        const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
        const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
        x = (__lane_id() < 32) ? a : b;
    }
    if constexpr (L == 64) {
        const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16));
        const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48));
        x = max(a, b);
    }
    return x;
}

// ---------------------------------------------------------------------------
// division: n = x / a correctly rounded from a per-block reciprocal
// ---------------------------------------------------------------------------

// r = RN(1/a) (IEEE division, once per block); q = RN(x r); e = x - q a
// (exact, fused); RN(q + e r) is the correctly rounded x / a (Markstein 1990,
// for a correctly rounded reciprocal and a first quotient within 1 ulp).
// Valid while no intermediate leaves the normal range; callers use it for
// 2^-60 <= a <= 2^60 and fall back to IEEE division otherwise.
__device__ __forceinline__ float div_by_block(float x, float a, float r)
{
    float q = x * r;
    float e = __builtin_fmaf(-q, a, x);
    return __builtin_fmaf(e, r, q);
}

// div_by_block of an fp16 x, read by the first two operations as a
// mixed-precision operand.  x * r is taken as a fused multiply-add onto +0:
// the same product except that -0 becomes +0, which div_by_block's result
// for x = -0 is anyway.
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float div_by_block_h(_Float16 x, float a, float r)
{
    const float q = __builtin_fmaf((float)x, r, 0.0f);
    const float e = __builtin_fmaf(-q, a, (float)x);
    return __builtin_fmaf(e, r, q);
}

__device__ __forceinline__ bool fast_div_ok(float a)
{
    return a >= 0x1p-60f && a <= 0x1p60f;
}

// n = x / a as every encoder takes it (|x| <= a): the correctly rounded
// quotient, 0 when a == 0.  `fast` = fast_div_ok(a), r = rcp_rn(a), both once
// per block.
__device__ __forceinline__ float normalize_by_block(float x, float a, float r, bool fast)
{
    return fast ? div_by_block(x, a, r) : (a > 0.0f ? x / a : 0.0f);
}

// RN(1/a) for 2^-60 <= a <= 2^60: the hardware reciprocal (about 1 ulp) and
// one Newton step with fused multiply-adds.  Checked on gfx950 against the
// IEEE quotient 1.0f / a for every significand at exponents -60, -20, -1, 0,
// 1, 20 and 60 (no difference); the significand of the result does not
// depend on the exponent of a in this range.
__device__ __forceinline__ float rcp_rn(float a)
{
    const float r0 = __builtin_amdgcn_rcpf(a);
    const float e = __builtin_fmaf(-a, r0, 1.0f);
    return __builtin_fmaf(e, r0, r0);
}

// ---------------------------------------------------------------------------
// encoders (tables staged in LDS)
// ---------------------------------------------------------------------------

// Copies WORDS dwords from global memory to LDS with NT threads in two
// phases: load() reads this thread's words into registers (an index past the
// end re-reads the last word), store() writes those in range.  Calling the
// load() of every table, then hold() of every table, before any store() keeps
// all the loads in flight together, so the waves wait for them once (a load
// and its store one round at a time would wait once per round).
template <int NT, int WORDS>
struct StageWords {
    static constexpr int R = (WORDS + NT - 1) / NT;
    uint32_t v[R];
    __device__ __forceinline__ void load(const void* src, int tid)
    {
        const uint32_t* const s = static_cast<const uint32_t*>(src);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = r * NT + tid;
            v[r] = s[i < WORDS ? i : WORDS - 1];
        }
    }
    // No instruction: the words are in registers here, so the compiler can
    // neither sink a load into the branch of its store nor delay it.
    __device__ __forceinline__ void hold()
    {
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" : "+v"(v[r]));
    }
    __device__ __forceinline__ void store(void* dst, int tid) const
    {
        uint32_t* const d = static_cast<uint32_t*>(dst);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if ((r + 1) * NT <= WORDS || r * NT + tid < WORDS) d[r * NT + tid] = v[r];
    }
};

// LDS copy of the dynamic-code encoder.  The base-code table is indexed
// directly by (bits of the clamped |n|) >> 17, with the sign bit moved to bit
// 13: the used entries sit at [kDynBase, kDynBase + 1409) and the same plus
// 8192; the rest of the array is never read (it saves the index arithmetic).
constexpr int kDynIdxSign = 8192;
constexpr int kDynIdxBytes = kDynIdxSign + kDynBase + kDynBucketBytes;   // 16324

struct DynEncLds {
    uint32_t base[kDynIdxBytes / 4];
    float thr[256];
};

// Stage the encoder tables (about 3.8 KB used) into LDS with NT threads: all
// loads first, then all stores (one wait).
template <int NT = kThreads>
__device__ __forceinline__ void stage_dyn_enc(DynEncLds& s, const QbTables* __restrict__ tab, int tid)
{
    constexpr int W = kDynBucketBytes / 4;                     // 353 words per sign
    StageWords<NT, W> pos, neg;
    StageWords<NT, 256> thr;
    pos.load(&tab->dyn8_base[0][0], tid);
    neg.load(&tab->dyn8_base[1][0], tid);
    thr.load(tab->dyn8_thr, tid);
    pos.hold();
    neg.hold();
    thr.hold();
    pos.store(&s.base[kDynBase / 4], tid);
    neg.store(&s.base[(kDynIdxSign + kDynBase) / 4], tid);
    thr.store(s.thr, tid);
}

// Dynamic 8-bit code of a normalized value in [-1, 1].
__device__ __forceinline__ uint32_t enc_dyn8(float nv, const DynEncLds& s)
{
    const float cl = __builtin_amdgcn_fmed3f(__builtin_fabsf(nv), 0x1p-22f, 1.0f);
    const uint32_t idx = (fbits(cl) >> kDynShift) | ((fbits(nv) >> 31) << 13);
    const uint32_t c = reinterpret_cast<const uint8_t*>(s.base)[idx];
    return c + (nv >= s.thr[c] ? 1u : 0u);
}

// Same for a value known to be >= 0 (+0 included).
__device__ __forceinline__ uint32_t enc_dyn8_pos(float nv, const DynEncLds& s)
{
    const float cl = __builtin_amdgcn_fmed3f(nv, 0x1p-22f, 1.0f);
    const uint32_t c = reinterpret_cast<const uint8_t*>(s.base)[fbits(cl) >> kDynShift];
    return c + (nv >= s.thr[c] ? 1u : 0u);
}

// LDS copy of the unsigned dynamic-code encoder (n >= 0): the code at the start
// of each bucket of n (bits of the clamped n >> 16), and the 255 thresholds.
struct UDynEncLds {
    uint8_t base[kUDynBucketBytes];
    float thr[256];
};

// Unsigned dynamic 8-bit code of a normalized value in [0, 1].
__device__ __forceinline__ uint32_t enc_udyn8(float nv, const UDynEncLds& s)
{
    const float cl = __builtin_amdgcn_fmed3f(nv, 0x1p-22f, 1.0f);
    const uint32_t c = s.base[(fbits(cl) >> kUDynShift) - kUDynBase];
    return c + (nv >= s.thr[c] ? 1u : 0u);
}

// LDS copy of a user code's encoder: the thresholds and their bucket index.
struct UserEncLds {
    float thr[256];
    uint8_t first[kUserFirstBytes];
};

// 8-bit code of a user code: the number of thresholds <= nv.  Those of earlier
// buckets all count and those of later ones none, so only nv's own bucket is
// searched.  With at most one threshold there (every bucket of the linear
// code and of quantile codes with no entries crowded within 2^-11) one
// compare decides: thr[c] then lies in this bucket or a later one
// (thr[255] = +inf).  A crowded bucket takes a binary search over its own
// thresholds.
__device__ __forceinline__ uint32_t enc_user(float nv, const UserEncLds& s)
{
    const int b = user_bucket(nv);
    uint32_t c = s.first[b];
    const uint32_t m = s.first[b + 1] - c;            // thresholds thr[c .. c+m) in bucket b
    if (m > 1) {
        uint32_t len = m;
        while (len != 0) {
            const uint32_t h = len >> 1;
            if (nv >= s.thr[c + h]) {
                c += h + 1;
                len -= h + 1;
            } else {
                len = h;
            }
        }
    } else {
        c += nv >= s.thr[c] ? 1u : 0u;
    }
    return c;
}

// Stage a user code's encoder into LDS with NT threads (one wait).
template <int NT = kThreads>
__device__ __forceinline__ void stage_user_enc(UserEncLds& s, const UserCode* __restrict__ code, int tid)
{
    StageWords<NT, 256> thr;
    StageWords<NT, kUserFirstBytes / 4> fst;
    thr.load(code->thr, tid);
    fst.load(code->first, tid);
    thr.hold();
    fst.hold();
    thr.store(s.thr, tid);
    fst.store(s.first, tid);
}

// 4-bit code of a normalized value in [-1, 1] from the bucket table in LDS:
// bucket k = 16 nv + 16 rounded to the nearest integer, ties to even, in
// [0, 32] (one fused multiply-add onto 1.5 * 2^23: the sum's float bits are
// 0x4B400000 + k, so one shift-and-add gives the entry's byte address), then
// below or above the bucket's one threshold.  NF4 (codes ascend with the
// values): the payload is the code below, the code above is one more.  FP4:
// the payload holds the code below in byte 0 and the one above in byte 1.
// |nv| <= 1 holds for every finite input (nv = x / absmax).
__device__ __forceinline__ const uint2& lut4_entry(float nv, const uint2* __restrict__ lut)
{
    const uint32_t t = fbits(__builtin_fmaf(nv, 16.0f, 0x1.8p23f + 16.0f));
    const uint32_t off = (t << 3) - (0x4B400000u << 3);            // 8 k (mod 2^32)
    return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(lut) + off);
}

__device__ __forceinline__ uint32_t enc_nf4(float nv, const uint2* __restrict__ lut)
{
    const uint2 e = lut4_entry(nv, lut);
    return e.y + (nv >= ffrom(e.x) ? 1u : 0u);
}

__device__ __forceinline__ uint32_t enc_fp4(float nv, const uint2* __restrict__ lut)
{
    const uint2 e = lut4_entry(nv, lut);
    return __builtin_amdgcn_ubfe(e.y, nv >= ffrom(e.x) ? 8u : 0u, 8u);
}

}  // namespace qb
