// qb_dequant.hip -- block-wise dequantization (8-bit dynamic code, 4-bit NF4 /
// FP4 packed two per byte), with the nested absmax decoded in the same pass.
//
// Method: element i of block b comes back as code[c_i] times the block's
// absmax, rounded once to the output dtype ("Bitsandbytes", section on
// dequantizing; compute dtype: "Quantize 🤗 Transformers models", section
// Change the compute dtype).  With nested quantization the absmax itself is
// decoded first, a_b = dyn8[c2_b] * absmax2[b / B2] + mean, two rounded binary32
// operations ("Bitsandbytes", section İç içe nicelleştirme).
//
// Kernel shape: one 256-thread workgroup per tile of 8192 elements for 4-bit
// codes and 4096 (2048 into binary32) for 8-bit codes (the best measured on
// MI355X), in tile order.  A thread takes units
// of E consecutive elements, E = 16 bytes of output (8 for 16-bit outputs, 4
// for fp32), consecutive lanes on consecutive units, so every load and store
// instruction of a wave covers one contiguous span.
// At the start a workgroup issues the loads of its codes and of the scale
// inputs of its tile's blocks (one block per thread, at most 128 blocks per
// tile since B >= 64), then stages the code tables in LDS; the blocks' scales
// are decoded once into LDS, and every element is one LDS lookup, one multiply
// and a round-to-nearest-even store.  Streamed codes and outputs take
// non-temporal accesses.
//
// Many tensors go in one launch: tiles of all tensors are numbered in one
// range and a workgroup finds its tensor through the coarse bucket index.
#include "qb_device.h"

namespace qb {

namespace {

// XCD-contiguous tile order (tile_of) for grouped launches; measured on
// MI355X it speeds up the grouped 7B-weight sweep by about 3% and slows
// single-tensor launches by about 10%, so those keep the plain order.
#ifndef QB_DQ_MULTI_REMAP
#define QB_DQ_MULTI_REMAP 1
#endif
// Decode the nested absmax with the dynamic code read from global memory (L2)
// by the threads that own a block, instead of staging the whole code in LDS.
#ifndef QB_DQ_DIRECT_DYN
#define QB_DQ_DIRECT_DYN 0
#endif

constexpr int kDqThreads = 256;
static_assert(dequant_tile_elems(4, false, DT_BF16) / 64 <= kDqThreads &&
                  dequant_tile_elems(4, true, DT_BF16) / 64 <= kDqThreads &&
                  dequant_tile_elems(8, false, DT_BF16) / 64 <= kDqThreads &&
                  dequant_tile_elems(8, false, DT_F32) / 64 <= kDqThreads,
              "one thread per block of a tile");

// The E codes of the unit at element offset e (a multiple of E) from base:
// E * BITS / 8 bytes (2, 4 or 8).
template <int BITS, int E>
__device__ __forceinline__ u32x2 load_unit(const uint8_t* base, uint32_t e)
{
    constexpr int bytes = E * BITS / 8;
    if constexpr (bytes == 8) {
        return gldo<u32x2>(base, e);
    } else if constexpr (bytes == 4) {
        u32x2 w = {gldo<uint32_t>(base, e * BITS / 8), 0u};
        return w;
    } else {
        u32x2 w = {(uint32_t)gldo<uint16_t>(base, e * BITS / 8), 0u};
        return w;
    }
}

// Code of element j (0 .. E-1) of a unit.
template <int BITS>
__device__ __forceinline__ uint32_t unit_code(const u32x2& w, int j)
{
    if constexpr (BITS == 8) {
        return ((j < 4 ? w.x : w.y) >> (8 * (j & 3))) & 0xFFu;
    } else {
        // byte k holds element 2k in its high nibble and 2k+1 in its low one
        const uint32_t byte = (w.x >> (8 * (j >> 1))) & 0xFFu;
        return (j & 1) ? (byte & 15u) : (byte >> 4);
    }
}

// Code of element idx of a tensor (scalar path of the last tile).
template <int BITS>
__device__ __forceinline__ uint32_t elem_code(const uint8_t* codes, int64_t idx)
{
    if constexpr (BITS == 8) {
        return gld<uint8_t>(codes + idx);
    } else {
        const uint32_t byte = gld<uint8_t>(codes + idx / 2);
        return (idx & 1) ? (byte & 15u) : (byte >> 4);
    }
}

// USER: 8-bit codes of a user code (`user`) instead of the dynamic code.
template <int BITS, int YDT, bool DQ, bool MULTI, bool USER = false>
__global__ __launch_bounds__(kDqThreads) void k_dequant(DequantDesc single, TileMap<DequantDesc> map, int log2B,
                                                        int log2B2, int code4, const QbTables* __restrict__ tab,
                                                        const UserCode* __restrict__ user)
{
    static_assert(!USER || (BITS == 8 && !DQ), "user codes are 8-bit, without nesting");
    __shared__ float s_val[BITS == 8 ? 256 : 16];   // decode table of the codes
    __shared__ float s_dyn[DQ && BITS == 4 && !QB_DQ_DIRECT_DYN ? 256 : 1];
    // a unit is E elements whose output a lane writes with one 16-byte store
    constexpr int E = YDT == DT_F32 ? 4 : 8;
    constexpr int kDqElems = (int)dequant_tile_elems(BITS, MULTI, YDT);
    static_assert(kDqElems % (kDqThreads * E) == 0, "whole units per thread");
    constexpr int kDqUnits = kDqElems / (kDqThreads * E);                // units per thread
    __shared__ float s_scale[kDqElems / 64];                            // blocks per tile at B = 64
    const int tid = threadIdx.x;
    const int64_t tile = tile_of<MULTI && QB_DQ_MULTI_REMAP>(blockIdx.x, gridDim.x);

    DequantDesc d;
    int64_t lt;
    if constexpr (MULTI) {
        d = map.descs[find_tensor(map, tile)];
        lt = tile - d.tile_begin;
    } else {
        d = single;
        lt = tile;
    }
    const int64_t n = d.n;
    const int64_t tbase = lt * kDqElems;                 // first element of the tile
    const bool full = tbase + kDqElems <= n;
    const uint8_t* const ct = d.codes + (tbase * BITS) / 8;

    // codes of the tile
    u32x2 w[kDqUnits];
    if (full) {
#pragma unroll
        for (int k = 0; k < kDqUnits; ++k) w[k] = load_unit<BITS, E>(ct, (uint32_t)(k * kDqThreads + tid) * E);
    }
    // scale inputs of the tile's blocks, one block per thread (B and the tile
    // are powers of two: a tile holds whole blocks, or lies within one block)
    const int nbt = (kDqElems >> log2B) > 0 ? (kDqElems >> log2B) : 1;
    const int64_t blk = (tbase >> log2B) + tid;
    const int64_t nb = (n + (int64_t(1) << log2B) - 1) >> log2B;
    const bool owner = tid < nbt && blk < nb;
    float sa = 0.0f;
    uint32_t sc = 0;
    if (owner) {
        if constexpr (DQ) {
            sc = gld<uint8_t>(d.c2 + blk);
            sa = gld<float>(d.absmax2 + (blk >> log2B2));
            if constexpr (BITS == 4 && QB_DQ_DIRECT_DYN) sa = tab->dyn8[sc] * sa;
        } else {
            sa = gld<float>(d.absmax + blk);
        }
    }
    const float mu = DQ ? gld<float>(d.offset) : 0.0f;

    // decode tables
    if constexpr (USER) {
        s_val[tid] = user->values[tid];
    } else if constexpr (BITS == 8) {
        s_val[tid] = tab->dyn8[tid];
    } else {
        // Every thread reads its words of both tables (the 16 code values at
        // tid % 16) before any is stored: the loads are in flight together
        // and the waves wait once, not once per table.
        float tv = (code4 == 0 ? tab->nf4 : tab->fp4)[tid & 15];
        float td = 0.0f;
        if constexpr (DQ && !QB_DQ_DIRECT_DYN) td = tab->dyn8[tid];
        asm volatile("" : "+v"(tv), "+v"(td));      // no instruction: keeps the loads ahead of the stores
        if (tid < 16) s_val[tid] = tv;
        if constexpr (DQ && !QB_DQ_DIRECT_DYN) s_dyn[tid] = td;
    }
    __syncthreads();
    if (owner) {
        if constexpr (DQ) {
            const float prod = (BITS == 4 && QB_DQ_DIRECT_DYN) ? sa : (BITS == 8 ? s_val : s_dyn)[sc] * sa;
            s_scale[tid] = prod + mu;
        } else {
            s_scale[tid] = sa;
        }
    }
    __syncthreads();

    char* const yt = static_cast<char*>(d.y) + tbase * (YDT == DT_F32 ? 4 : 2);
    if (full) {
#pragma unroll
        for (int k = 0; k < kDqUnits; ++k) {
            const uint32_t e = (uint32_t)(k * kDqThreads + tid) * E;
            const float s = s_scale[e >> log2B];
            float o[E];
#pragma unroll
            for (int j = 0; j < E; ++j) o[j] = s_val[unit_code<BITS>(w[k], j)] * s;
            if constexpr (E == 4) store4o<YDT>(yt, e, o);
            else store8o<YDT>(yt, e, o);
        }
    } else {
        for (int k = 0; k < kDqUnits; ++k)
            for (int j = 0; j < E; ++j) {
                const uint32_t e = (uint32_t)(k * kDqThreads + tid) * E + j;
                if ((int64_t)e < n - tbase) {
                    const float s = s_scale[e >> log2B];
                    store1<YDT>(yt, e, s_val[elem_code<BITS>(ct, e)] * s);
                }
            }
    }
}

int ilog2(int v)
{
    int k = 0;
    while ((1 << k) < v) ++k;
    return k;
}

template <int BITS, int YDT, bool DQ>
hipError_t dequant_as(const DequantDesc& single, const TileMap<DequantDesc>* map, int64_t ntiles, int code4, int B,
                      int B2, const QbTables* tab, hipStream_t s)
{
    if (ntiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (map)
        return launch_kernel_nt(k_dequant<BITS, YDT, DQ, true>, (int)ntiles, kDqThreads, s, single, *map, ilog2(B),
                                ilog2(B2), code4, tab, (const UserCode*)nullptr);
    return launch_kernel_nt(k_dequant<BITS, YDT, DQ, false>, (int)ntiles, kDqThreads, s, single,
                            TileMap<DequantDesc>{}, ilog2(B), ilog2(B2), code4, tab, (const UserCode*)nullptr);
}

template <int BITS, bool DQ>
hipError_t dequant_y(int ydt, const DequantDesc& single, const TileMap<DequantDesc>* map, int64_t ntiles, int code4,
                     int B, int B2, const QbTables* tab, hipStream_t s)
{
    switch (ydt) {
    case DT_F32: return dequant_as<BITS, DT_F32, DQ>(single, map, ntiles, code4, B, B2, tab, s);
    case DT_F16: return dequant_as<BITS, DT_F16, DQ>(single, map, ntiles, code4, B, B2, tab, s);
    case DT_BF16: return dequant_as<BITS, DT_BF16, DQ>(single, map, ntiles, code4, B, B2, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_dequant_user(const DequantDesc& d, int64_t ntiles, int B, int ydt, const UserCode* code,
                               hipStream_t s)
{
    if (ntiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    if (B < 64 || B > 4096 || (B & (B - 1))) return hipErrorInvalidValue;
    const int lb = ilog2(B);
    const TileMap<DequantDesc> none{};
    switch (ydt) {
    case DT_F32:
        return launch_kernel_nt(k_dequant<8, DT_F32, false, false, true>, (int)ntiles, kDqThreads, s, d, none, lb, 0,
                                0, (const QbTables*)nullptr, code);
    case DT_F16:
        return launch_kernel_nt(k_dequant<8, DT_F16, false, false, true>, (int)ntiles, kDqThreads, s, d, none, lb, 0,
                                0, (const QbTables*)nullptr, code);
    case DT_BF16:
        return launch_kernel_nt(k_dequant<8, DT_BF16, false, false, true>, (int)ntiles, kDqThreads, s, d, none, lb,
                                0, 0, (const QbTables*)nullptr, code);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequant(const DequantDesc& single, const TileMap<DequantDesc>* map, int64_t ntiles, int bits,
                          int code4, int B, int B2, bool dq, int ydt, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (B < 64 || B > 4096 || (B & (B - 1))) return hipErrorInvalidValue;
    if (bits == 8)
        return dq ? dequant_y<8, true>(ydt, single, map, ntiles, code4, B, B2, tab, s)
                  : dequant_y<8, false>(ydt, single, map, ntiles, code4, B, B2, tab, s);
    if (bits == 4)
        return dq ? dequant_y<4, true>(ydt, single, map, ntiles, code4, B, B2, tab, s)
                  : dequant_y<4, false>(ydt, single, map, ntiles, code4, B, B2, tab, s);
    return hipErrorInvalidValue;
}

}  // namespace qb
