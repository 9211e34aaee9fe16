// qb_device.h -- device helpers shared by the libqb kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qb_tables.h"

namespace qb {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int kThreads = 256;   // every kernel runs 256-thread workgroups (4 waves)

__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float ffrom(uint32_t u) { return __uint_as_float(u); }

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

// 4 consecutive elements at element index i (16-byte aligned for fp32, 8 for 16-bit).
template <int DT>
__device__ __forceinline__ void load4(const void* __restrict__ base, int64_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
        v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
        uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
        if constexpr (DT == DT_BF16) {
            v[0] = bf16_lo(x.x); v[1] = bf16_hi(x.x); v[2] = bf16_lo(x.y); v[3] = bf16_hi(x.y);
        } else {
            v[0] = f16_lo(x.x); v[1] = f16_hi(x.x); v[2] = f16_lo(x.y); v[3] = f16_hi(x.y);
        }
    }
}

// 8 consecutive elements at element index i (16-byte aligned for every type).
template <int DT>
__device__ __forceinline__ void load8(const void* __restrict__ base, int64_t i, float* v)
{
    if constexpr (DT == DT_F32) {
        load4<DT_F32>(base, i, v);
        load4<DT_F32>(base, i + 4, v + 4);
    } else {
        uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
        uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = DT == DT_BF16 ? bf16_lo(w[k]) : f16_lo(w[k]);
            v[2 * k + 1] = DT == DT_BF16 ? bf16_hi(w[k]) : f16_hi(w[k]);
        }
    }
}

template <int DT>
__device__ __forceinline__ float load1(const void* __restrict__ base, int64_t i)
{
    if constexpr (DT == DT_F32) {
        return static_cast<const float*>(base)[i];
    } else {
        uint32_t h = static_cast<const uint16_t*>(base)[i];
        return DT == DT_BF16 ? bf16_lo(h) : f16_lo(h);
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
__device__ __forceinline__ void store1(void* __restrict__ base, int64_t i, float v)
{
    if constexpr (DT == DT_F32)
        static_cast<float*>(base)[i] = v;
    else
        static_cast<uint16_t*>(base)[i] = (uint16_t)to_half_bits<DT>(v);
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
    if constexpr (L >= 32) x = max(x, (uint32_t)__shfl_xor((int)x, 16));
    if constexpr (L >= 64) x = max(x, (uint32_t)__shfl_xor((int)x, 32));
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

__device__ __forceinline__ bool fast_div_ok(float a)
{
    return a >= 0x1p-60f && a <= 0x1p60f;
}

// ---------------------------------------------------------------------------
// encoders (tables staged in LDS)
// ---------------------------------------------------------------------------

// Dynamic 8-bit code of a normalized value in [-1, 1].
__device__ __forceinline__ uint32_t enc_dyn8(float nv, const uint2* __restrict__ lut)
{
    uint32_t bits = fbits(nv);
    uint32_t mag = bits & 0x7FFFFFFFu;
    uint32_t cl = min(max(mag, kDynLowBits), kOneBits);
    uint2 e = lut[(cl >> kDynShift) - kDynBase];
    int cp = (int)e.y + (mag >= e.x ? 1 : 0);          // 127 .. 255
    int cn = max(254 - cp, 0);                          // mirrored; -1.0 is not in the code
    return (uint32_t)((int)bits < 0 ? cn : cp);
}

// Same for a value known to be >= 0 (+0 included).
__device__ __forceinline__ uint32_t enc_dyn8_pos(float nv, const uint2* __restrict__ lut)
{
    uint32_t mag = fbits(nv);
    uint32_t cl = min(max(mag, kDynLowBits), kOneBits);
    uint2 e = lut[(cl >> kDynShift) - kDynBase];
    return e.y + (mag >= e.x ? 1u : 0u);
}

// 4-bit code (NF4 or FP4 by the table) of a normalized value in [-1, 1].
__device__ __forceinline__ uint32_t enc_4bit(float nv, const uint2* __restrict__ lut)
{
    float u = nv * 16.0f + 16.0f;
    int b = min((int)u, k4LutN - 1);
    uint2 e = lut[b];
    return (nv >= ffrom(e.x)) ? ((e.y >> 8) & 0xFFu) : (e.y & 0xFFu);
}

}  // namespace qb
