// qb_matmul.hip -- 4-bit weights dequantized inside the matrix product:
// y = x W^T with W held as NF4 / FP4 codes (two per byte) and a block absmax
// (plain, or nested).
//
// A layer whose weights are stored in 4 bits computes in the compute dtype
// (bf16, fp16, or the default fp32): the weights come back to that dtype and
// multiply the activations ("Bitsandbytes", section QLoRA: Hesaplama veri
// türü; "Quantize 🤗 Transformers models", section Change the compute dtype).
// Each weight is dequantized exactly as by qb_dequantize into the compute
// dtype (code value times the block absmax, one binary32 multiply, one
// rounding), so the product is x times that matrix; only the order of the
// binary32 additions is the kernel's own.
//
// Shape (one workgroup of 8 waves per 16 output columns n and up to 64 rows m):
// a lane owns weight row n0 + (lane % 16) and, per step of 128 k, the 32
// consecutive k of its lane group (lane / 16): one 16-byte load of codes, one
// block absmax.  Those 32 dequantized weights feed four 16x16x32 MFMAs
// directly as B operands (a lane's eight k per MFMA are consecutive in W's
// rows, so W never goes through LDS); the activations are loaded in the same
// k order as A operands.  The 8 waves take the steps of K in turn, and their
// 16x16 partial sums are added in wave order through LDS: no second pass,
// and the same bits on every run.  The weights stream once from HBM (0.5
// byte per weight plus the absmax); the activations are re-read from L2 by
// every workgroup, which is cheap while M is small, the regime where a
// 4-bit layer is bound by reading its weights.
#include "qb_device.h"

namespace qb {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Steps of a wave whose loads are issued ahead of its computation.  Some of
// them are skipped on some paths (a step past the end, a row past M), so the
// compiler cannot count the loads in flight and waits for all of them before
// each step: the steps arrive in batches, not as a pipeline.  Measured on
// MI355X (kernel trace, 7B projection shapes, M = 1 .. 64): 2 beats 4 by up
// to 25% on the 11008-row layer (fewer registers: two workgroups per CU) and
// ties elsewhere.  A version with exact waits (every path issuing the same
// loads, rows past M read as bounds-checked buffer loads) at depths 2 to 6
// measured within 10% at M <= 16 and up to 15% slower at M >= 64: at these
// sizes the launch, the first HBM round trip and the dequantize instructions
// bound the kernel, not the depth.
#ifndef QB_MM_DEPTH
#define QB_MM_DEPTH 2
#endif

// Waves per workgroup: they share one tile of 16 output columns and take the
// steps of K in turn.  Measured on MI355X: 4 is up to 45% slower on the
// 11008-deep layer; 16 is 11% faster there but 9% slower on the 11008-row
// layer; 8 is the best compromise.
#ifndef QB_MM_WAVES
#define QB_MM_WAVES 8
#endif

constexpr int kMmWaves = QB_MM_WAVES;
constexpr int kMmThreads = 64 * kMmWaves;
constexpr int kMmStepK = 128;                // k per wave step: 4 lane groups x 32

// Eight weights or activations of one MFMA operand, in the compute dtype.
template <int XDT>
struct Frag {
    uint32_t w[4];                           // 8 x 16 bits (bf16 / fp16)
};
template <>
struct Frag<DT_F32> {
    float w[8];
};

template <int XDT>
__device__ __forceinline__ void frag_zero(Frag<XDT>& f)
{
#pragma unroll
    for (int i = 0; i < (XDT == DT_F32 ? 8 : 4); ++i) f.w[i] = 0;
}

// A T at byte offset off (uint32) from a uniform base: the address is the
// scalar base plus one 32-bit lane offset.  Cached (the activations and the
// block constants are re-read by other workgroups).
template <class T>
__device__ __forceinline__ T ldo(const void* base, uint32_t off)
{
    const QB_G char* const b = (const QB_G char*)base;          // global address space first
    return *(const QB_G T*)(b + off);
}

// Eight consecutive activations at element offset e (a multiple of 8) of x.
template <int XDT>
__device__ __forceinline__ void load_frag(const void* x, int64_t e, Frag<XDT>& f)
{
    if constexpr (XDT == DT_F32) {
        const f32x4 a = gld<f32x4>(static_cast<const float*>(x) + e);
        const f32x4 b = gld<f32x4>(static_cast<const float*>(x) + e + 4);
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
        f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
    } else {
        const u32x4 a = gld<u32x4>(static_cast<const uint16_t*>(x) + e);
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
    }
}

// Eight activations at byte offset off from a uniform base.
template <int XDT>
__device__ __forceinline__ void load_frag_o(const void* base, uint32_t off, Frag<XDT>& f)
{
    if constexpr (XDT == DT_F32) {
        const f32x4 a = ldo<f32x4>(base, off), b = ldo<f32x4>(base, off + 16u);
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
        f.w[4] = b.x; f.w[5] = b.y; f.w[6] = b.z; f.w[7] = b.w;
    } else {
        const u32x4 a = ldo<u32x4>(base, off);
        f.w[0] = a.x; f.w[1] = a.y; f.w[2] = a.z; f.w[3] = a.w;
    }
}

// acc += A B over the 8 k of this lane's fragments (16x16 tile).
template <int XDT>
__device__ __forceinline__ void mma(const Frag<XDT>& a, const Frag<XDT>& b, f32x4& acc)
{
    if constexpr (XDT == DT_BF16) {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a.w, 16);
        __builtin_memcpy(&bv, b.w, 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    } else if constexpr (XDT == DT_F16) {
        f16x8 av, bv;
        __builtin_memcpy(&av, a.w, 16);
        __builtin_memcpy(&bv, b.w, 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
    } else {
        // binary32: eight 16x16x4 products, one k per lane group each
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w[i], b.w[i], acc, 0, 0, 0);
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two binary32 values rounded to nearest even into one word of the compute
// dtype, a in the low half.
template <int XDT>
__device__ __forceinline__ uint32_t pack_pair(float a, float b)
{
    if constexpr (XDT == DT_BF16) {
        const bf16x2 h = __builtin_convertvector((f32x2{a, b}), bf16x2);    // one v_cvt_pk_bf16_f32
        uint32_t u;
        __builtin_memcpy(&u, &h, 4);
        return u;
    } else {
        return pack2<XDT>(a, b);
    }
}

// The 32 weights of a lane's chunk: code value times the block absmax, one
// binary32 multiply, rounded once to the compute dtype (as qb_dequantize).
// Byte j of a code word holds element 2j (high nibble) and 2j+1 (low); two
// masks per word turn all eight nibbles into byte offsets into the 16-entry
// table of code values in LDS.
template <int XDT>
__device__ __forceinline__ void dequant_chunk(const u32x4& cw, float a, const float* s_val, Frag<XDT>* f)
{
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    const char* const tv = reinterpret_cast<const char*>(s_val);
#pragma unroll
    for (int q = 0; q < 4; ++q) {                  // fragment q: bytes 4q .. 4q+3 of the chunk
        uint32_t th = (words[q] >> 2) & 0x3C3C3C3Cu;           // 4 * high nibbles
        uint32_t tl = (words[q] << 2) & 0x3C3C3C3Cu;           // 4 * low nibbles
        // Opaque to the compiler (no instruction): it would otherwise fold
        // the masks into a shift and a mask per nibble, where one bit-field
        // extract per nibble suffices.
        asm("" : "+v"(th), "+v"(tl));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float hi = *reinterpret_cast<const float*>(tv + __builtin_amdgcn_ubfe(th, 8 * j, 8)) * a;
            const float lo = *reinterpret_cast<const float*>(tv + __builtin_amdgcn_ubfe(tl, 8 * j, 8)) * a;
            if constexpr (XDT == DT_F32) {
                f[q].w[2 * j] = hi;
                f[q].w[2 * j + 1] = lo;
            } else {
                f[q].w[j] = pack_pair<XDT>(hi, lo);
            }
        }
    }
}

template <int XDT, bool DQ, int MT, bool KF>
__global__ __launch_bounds__(kMmThreads) void k_dq4_matmul(const void* __restrict__ x, int64_t M, int64_t K,
                                                           const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ absmax,
                                                           const uint8_t* __restrict__ c2,
                                                           const float* __restrict__ absmax2,
                                                           const float* __restrict__ offset, int log2B, int log2B2,
                                                           int code4, int64_t N, void* __restrict__ y,
                                                           const QbTables* __restrict__ tab)
{
    __shared__ float s_val[16];
    __shared__ float s_dyn[DQ ? 256 : 1];
    __shared__ float s_red[kMmWaves][MT][4][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: scalar step bases
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16 * MT;
    // Weight rows past N read row N - 1 instead (their outputs are never
    // stored); activation rows past M are not loaded and stay zero.
    constexpr int ES = XDT == DT_F32 ? 4 : 2;         // bytes per activation
    const int rn = n0 + r < N ? r : (int)(N - 1 - n0);
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // Uniform bases of the workgroup's tile (step s adds s * 64 code bytes,
    // s * 2 block constants at B = 64, s * 128 activations); per-lane 32-bit
    // offsets fixed for the whole loop.
    const uint8_t* const cw_base = codes + n0 * K / 2;
    const uint32_t cw_off = (uint32_t)(rn * K / 2 + 16 * g);
    const int64_t e_tile = n0 * K;                    // element index of the tile's first weight
    const uint32_t e_lane = (uint32_t)(rn * K + 32 * g);
    const char* const x_base = static_cast<const char*>(x) + m0 * K * ES;
    bool m_ok[MT];
    uint32_t x_off[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        m_ok[t] = m0 + 16 * t + r < M;
        x_off[t] = (uint32_t)(((16 * t + r) * K + 32 * g) * ES);
    }

    // The loads of a wave's next PD steps (codes, block constants, and with
    // one m-tile the activations too) are issued ahead of the current step's
    // computation.
    constexpr bool PX = MT == 1;
    constexpr int PD = (XDT == DT_F32 && PX) ? 2 : QB_MM_DEPTH;
    struct Pre {
        u32x4 cw;
        uint32_t c;
        float a;
        Frag<XDT> xf[PX ? 4 : 1];
    };
    const int64_t steps = (K + kMmStepK - 1) / kMmStepK;
    float mu = 0.0f;                                  // the nested mean, read with the tables
    // a lane group's 32 k lie inside K, except in the last step when K is not
    // a multiple of 128 (KF false): such a lane feeds zeros instead
    auto in_k = [&](int64_t s) { return KF || s * kMmStepK + 32 * g < K; };
    auto issue = [&](Pre& p, int64_t s) {
        if (s >= steps) return;
        if (!in_k(s)) return;
        p.cw = ldo<u32x4>(cw_base + s * (kMmStepK / 2), cw_off);
        const int64_t blk = (e_tile + s * kMmStepK + e_lane) >> log2B;
        if constexpr (DQ) {
            p.c = gld<uint8_t>(c2 + blk);
            p.a = gld<float>(absmax2 + (blk >> log2B2));
        } else {
            p.a = gld<float>(absmax + blk);
        }
        if constexpr (PX) {
            if (m_ok[0]) {
                const char* const xs = x_base + s * kMmStepK * ES;
#pragma unroll
                for (int q = 0; q < 4; ++q) load_frag_o<XDT>(xs, x_off[0] + (uint32_t)(8 * ES) * q, p.xf[q]);
            }
        }
    };
    auto compute = [&](Pre& p, int64_t s) {
        const bool kin = in_k(s);
        Frag<XDT> b[4];
        if (kin) {
            const float a = DQ ? s_dyn[p.c] * p.a + mu : p.a;    // two rounded operations (nested)
            dequant_chunk<XDT>(p.cw, a, s_val, b);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) frag_zero<XDT>(b[q]);
        }
        if constexpr (PX) {
            if (!kin) {
#pragma unroll
                for (int q = 0; q < 4; ++q) frag_zero<XDT>(p.xf[q]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) mma<XDT>(p.xf[q], b[q], acc[0]);
        } else {
            const char* const xs = x_base + s * kMmStepK * ES;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                Frag<XDT> xa[4];
                if (m_ok[t] && kin) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) load_frag_o<XDT>(xs, x_off[t] + (uint32_t)(8 * ES) * q, xa[q]);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) frag_zero<XDT>(xa[q]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) mma<XDT>(xa[q], b[q], acc[t]);
            }
        }
    };
    Pre pre[PD];
#pragma unroll
    for (int j = 0; j < PD; ++j) {
        if constexpr (PX) {
#pragma unroll
            for (int q = 0; q < 4; ++q) frag_zero<XDT>(pre[j].xf[q]);
        }
        issue(pre[j], wave + (int64_t)kMmWaves * j);
    }
    // the code tables are staged while the first steps' loads are in flight
    if (tid < 16) s_val[tid] = (code4 == 0 ? tab->nf4 : tab->fp4)[tid];
    if constexpr (DQ) {
        if (tid < 256) s_dyn[tid] = tab->dyn8[tid];
    }
    mu = DQ ? gld<float>(offset) : 0.0f;
    __syncthreads();
    for (int64_t base = wave; base < steps; base += (int64_t)kMmWaves * PD) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const int64_t s = base + (int64_t)kMmWaves * j;
            if (s < steps) compute(pre[j], s);
            issue(pre[j], s + (int64_t)kMmWaves * PD);
        }
    }

    // add the waves' partial tiles in wave order
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_red[wave][t][j][lane] = acc[t][j];
    __syncthreads();
    for (int o = tid; o < MT * 256; o += kMmThreads) {
        const int ml = o >> 4, nl = o & 15;               // consecutive threads: consecutive n
        const int t = ml >> 4, mm = ml & 15;
        const int l = (mm >> 2) * 16 + nl, j = mm & 3;    // C[m][n] of the 16x16 tile: lane, element
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kMmWaves; ++w) sum += s_red[w][t][j][l];
        const int64_t m = m0 + ml, nn = n0 + nl;
        if (m < M && nn < N) store1<XDT>(y, m * N + nn, sum);
    }
}

// Enqueue `kernel` on a 2-D grid of kMmThreads-thread workgroups; returns
// this launch's own status.
template <typename... KArgs, typename... Args>
hipError_t launch_2d(void (*kernel)(KArgs...), dim3 grid, hipStream_t s, Args&&... args)
{
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kMmThreads), ptrs, 0, s);
        },
        vals);
}

template <int XDT, bool DQ, int MT>
hipError_t mm_as(const void* x, int64_t M, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    const int64_t gx = (N + 15) / 16, gy = (M + 16 * MT - 1) / (16 * MT);
    if (gx >= (int64_t(1) << 31) || gy > 65535) return hipErrorInvalidValue;
    if (K % kMmStepK == 0)
        return launch_2d(k_dq4_matmul<XDT, DQ, MT, true>, dim3((unsigned)gx, (unsigned)gy), s, x, M, K, codes,
                         absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab);
    return launch_2d(k_dq4_matmul<XDT, DQ, MT, false>, dim3((unsigned)gx, (unsigned)gy), s, x, M, K, codes, absmax,
                     c2, absmax2, offset, log2B, log2B2, code4, N, y, tab);
}

template <int XDT, bool DQ>
hipError_t mm_mt(int64_t M, const void* x, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    if (M <= 16) return mm_as<XDT, DQ, 1>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    if (M <= 32) return mm_as<XDT, DQ, 2>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    return mm_as<XDT, DQ, 4>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
}

}  // namespace

hipError_t launch_dq4_matmul(const void* x, int xdt, int64_t M, int64_t K, const uint8_t* codes, const float* absmax,
                             const uint8_t* c2, const float* absmax2, const float* offset, int B, int B2, int code4,
                             int64_t N, void* y, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    int log2B = 0, log2B2 = 0;
    while ((1 << log2B) < B) ++log2B;
    while ((1 << log2B2) < B2) ++log2B2;
    const bool dq = c2 != nullptr;
    switch (xdt) {
    case DT_BF16:
        return dq ? mm_mt<DT_BF16, true>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s)
                  : mm_mt<DT_BF16, false>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    case DT_F16:
        return dq ? mm_mt<DT_F16, true>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s)
                  : mm_mt<DT_F16, false>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    case DT_F32:
        return dq ? mm_mt<DT_F32, true>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s)
                  : mm_mt<DT_F32, false>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qb
