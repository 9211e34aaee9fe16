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

constexpr int kMmWaves = 8;
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

// The 32 weights of a lane's chunk: code value times the block absmax, one
// binary32 multiply, rounded once to the compute dtype (as qb_dequantize).
template <int XDT>
__device__ __forceinline__ void dequant_chunk(const u32x4& cw, float a, const float* s_val, Frag<XDT>* f)
{
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {                  // fragment q: bytes 4q .. 4q+3 of the chunk
#pragma unroll
        for (int j = 0; j < 4; ++j) {              // byte j: element 2j in the high nibble, 2j+1 in the low
            const uint32_t byte = (words[q] >> (8 * j)) & 0xFFu;
            const float hi = s_val[byte >> 4] * a;
            const float lo = s_val[byte & 15u] * a;
            if constexpr (XDT == DT_F32) {
                f[q].w[2 * j] = hi;
                f[q].w[2 * j + 1] = lo;
            } else {
                f[q].w[j] = pack2<XDT>(hi, lo);
            }
        }
    }
}

template <int XDT, bool DQ, int MT>
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16, m0 = (int64_t)blockIdx.y * 16 * MT;
    if (tid < 16) s_val[tid] = (code4 == 0 ? tab->nf4 : tab->fp4)[tid];
    if constexpr (DQ) {
        if (tid < 256) s_dyn[tid] = tab->dyn8[tid];
    }
    const float mu = DQ ? gld<float>(offset) : 0.0f;
    __syncthreads();

    const int64_t n = n0 + r;
    const bool row_ok = n < N;
    f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t steps = (K + kMmStepK - 1) / kMmStepK;
    for (int64_t s = wave; s < steps; s += kMmWaves) {
        const int64_t kk = s * kMmStepK + 32 * g;        // this lane's first k
        const bool k_ok = kk < K;
        Frag<XDT> b[4];
        if (row_ok && k_ok) {
            const int64_t e = n * K + kk;                 // element index in W (a multiple of 32)
            const u32x4 cw = gld<u32x4>(codes + e / 2);
            const int64_t blk = e >> log2B;
            float a;
            if constexpr (DQ) {
                const float prod = s_dyn[gld<uint8_t>(c2 + blk)] * gld<float>(absmax2 + (blk >> log2B2));
                a = prod + mu;
            } else {
                a = gld<float>(absmax + blk);
            }
            dequant_chunk<XDT>(cw, a, s_val, b);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) frag_zero<XDT>(b[q]);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int64_t m = m0 + 16 * t + r;
            Frag<XDT> a[4];
            if (m < M && k_ok) {
#pragma unroll
                for (int q = 0; q < 4; ++q) load_frag<XDT>(x, m * K + kk + 8 * q, a[q]);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) frag_zero<XDT>(a[q]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) mma<XDT>(a[q], b[q], acc[t]);
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
    return launch_2d(k_dq4_matmul<XDT, DQ, MT>, dim3((unsigned)gx, (unsigned)gy), s, x, M, K, codes, absmax, c2,
                     absmax2, offset, log2B, log2B2, code4, N, y, tab);
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
