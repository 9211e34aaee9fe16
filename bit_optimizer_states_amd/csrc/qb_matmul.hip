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

// A few rows of activations (decode), 16-bit, M * K * 2 bytes at most this
// many (K rounded up to whole steps of 128 k): the rows are staged in LDS once
// per workgroup (dynamic LDS, zero past K), so no activation registers are
// held per step and x is not fetched again from L2 every step.  The freed
// registers go to occupancy: the code loads of one step are in flight per
// wave where a wave has at most 4 steps of K, two steps beyond (same-process
// A/B on the 7B projections at M = 1: q/k/v in one launch 13.8 -> 10.8 us,
// gate/up 22.5 -> 17.0 us; the 11008-deep layer 11.1 -> 10.9 us with two;
// at M = 4 against x from L2 every step: q/k/v 15.2 -> 10.6 us, gate/up
// 26.0 -> 18.9 us; at M = 8, 64 KiB against 32: q/k/v 17.2 -> 15.1 us,
// gate/up 29.2 -> 24.3 us.  Staging 16 rows, 128 KiB, leaves one workgroup
// per CU and is 10-40% slower at M = 12 and 16).
#ifndef QB_MM_XS_BYTES
#define QB_MM_XS_BYTES 65536
#endif
// Rows of activations staged this way: up to this many (each row padded by
// 64 bytes, so the rows of one 16-byte fragment fall in different LDS banks).
#ifndef QB_MM_XS_ROWS
#define QB_MM_XS_ROWS 8
#endif
constexpr int kXsPad = 4;                     // u32x4 of padding per staged row

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
// Fragment q (bytes 4q .. 4q+3 of a lane's 16-byte chunk): eight weights.
template <int XDT>
__device__ __forceinline__ void dequant_frag(uint32_t word, float a, const float* s_val, Frag<XDT>& f)
{
    const char* const tv = reinterpret_cast<const char*>(s_val);
    uint32_t th = (word >> 2) & 0x3C3C3C3Cu;           // 4 * high nibbles
    uint32_t tl = (word << 2) & 0x3C3C3C3Cu;           // 4 * low nibbles
    // Opaque to the compiler (no instruction): it would otherwise fold the
    // masks into a shift and a mask per nibble, where one bit-field extract
    // per nibble suffices.
    asm("" : "+v"(th), "+v"(tl));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float hi = *reinterpret_cast<const float*>(tv + __builtin_amdgcn_ubfe(th, 8 * j, 8)) * a;
        const float lo = *reinterpret_cast<const float*>(tv + __builtin_amdgcn_ubfe(tl, 8 * j, 8)) * a;
        if constexpr (XDT == DT_F32) {
            f.w[2 * j] = hi;
            f.w[2 * j + 1] = lo;
        } else {
            f.w[j] = pack_pair<XDT>(hi, lo);
        }
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
    dequant_frag<XDT>(cw.x, a, s_val, f[0]);
    dequant_frag<XDT>(cw.y, a, s_val, f[1]);
    dequant_frag<XDT>(cw.z, a, s_val, f[2]);
    dequant_frag<XDT>(cw.w, a, s_val, f[3]);
}

// One workgroup's tile: output columns 16 ntile .. 16 ntile + 15 of y, rows
// 16 MT blockIdx.y onwards.
template <int XDT, bool DQ, int MT, bool KF, int XS>
__device__ __forceinline__ void mm_tile(const void* __restrict__ x, int64_t M, int64_t K,
                                        const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
                                        const uint8_t* __restrict__ c2, const float* __restrict__ absmax2,
                                        const float* __restrict__ offset, int log2B, int log2B2, int code4, int64_t N,
                                        void* __restrict__ y, const QbTables* __restrict__ tab, int64_t ntile)
{
    static_assert(XS == 0 || (MT == 1 && XDT != DT_F32), "staged activations: 16-bit rows of one m-tile");
    __shared__ float s_val[16];
    __shared__ float s_dyn[DQ ? 256 : 1];
    __shared__ float s_red[kMmWaves][MT][4][64];
    extern __shared__ u32x4 s_x[];                    // XS: the activation rows, whole steps (dynamic)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // uniform: scalar step bases
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = ntile * 16, m0 = (int64_t)blockIdx.y * 16 * MT;
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
    constexpr bool PX = MT == 1 && XS == 0;
    constexpr int PD = XS ? XS : ((XDT == DT_F32 && PX) ? 2 : QB_MM_DEPTH);
    struct Pre {
        u32x4 cw;
        uint32_t c;
        float a;
        Frag<XDT> xf[PX ? 4 : 1];
    };
    // XS: the step's activations, in lanes r < M (the rows of the tile); the
    // other lanes' fragments stay zero for the whole loop
    Frag<XDT> xr[XS ? 4 : 1];
#pragma unroll
    for (int q = 0; q < (XS ? 4 : 1); ++q) frag_zero<XDT>(xr[q]);
    const int64_t steps = (K + kMmStepK - 1) / kMmStepK;
    const int xs_rs = (int)steps * (kMmStepK / 8) + kXsPad;     // XS: u32x4 per staged row
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
        if constexpr (XS) {
            // activations of the step from LDS (zero past K): rows r < M
            if (m_ok[0]) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 v = s_x[r * xs_rs + s * (kMmStepK / 8) + 4 * g + q];
                    xr[q].w[0] = v.x;
                    xr[q].w[1] = v.y;
                    xr[q].w[2] = v.z;
                    xr[q].w[3] = v.w;
                }
            }
        }
        Frag<XDT> b[4];
        if (kin) {
            const float a = DQ ? s_dyn[p.c] * p.a + mu : p.a;    // two rounded operations (nested)
            dequant_chunk<XDT>(p.cw, a, s_val, b);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) frag_zero<XDT>(b[q]);
        }
        if constexpr (XS) {
#pragma unroll
            for (int q = 0; q < 4; ++q) mma<XDT>(xr[q], b[q], acc[0]);
        } else if constexpr (PX) {
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
    // the code tables (and the activation row) are staged while the first
    // steps' loads are in flight
    if constexpr (XS) {
        // M rows of whole steps: the chunks past K (K is a multiple of 32)
        // and the padding read as zero
        const int kc = (int)(K / 8);
        for (int i = tid; i < (int)M * xs_rs; i += kMmThreads) {
            const int row = i / xs_rs, c = i - row * xs_rs;
            s_x[i] = c < kc ? ldo<u32x4>(x_base, (uint32_t)((row * kc + c) * 16)) : u32x4{0u, 0u, 0u, 0u};
        }
    }
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

template <int XDT, bool DQ, int MT, bool KF, int XS>
__global__ __launch_bounds__(kMmThreads) void k_dq4_matmul(const void* __restrict__ x, int64_t M, int64_t K,
                                                           const uint8_t* __restrict__ codes,
                                                           const float* __restrict__ absmax,
                                                           const uint8_t* __restrict__ c2,
                                                           const float* __restrict__ absmax2,
                                                           const float* __restrict__ offset, int log2B, int log2B2,
                                                           int code4, int64_t N, void* __restrict__ y,
                                                           const QbTables* __restrict__ tab)
{
    mm_tile<XDT, DQ, MT, KF, XS>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab,
                                 (int64_t)blockIdx.x);
}

// Several weights against the same activations in one launch (the column
// tiles of weight i are tiles tile0[i] .. tile0[i + 1] - 1 of the grid's x
// dimension): the same tiles, bit for bit, as one launch per weight.
struct MmGroup {
    MmWeight w[kMmGroupMax];
    int64_t tile0[kMmGroupMax + 1];
    int count;
};

template <int XDT, bool DQ, int MT, bool KF, int XS>
__global__ __launch_bounds__(kMmThreads) void k_dq4_matmul_grouped(const void* __restrict__ x, int64_t M, int64_t K,
                                                                   const MmGroup grp, int log2B, int log2B2,
                                                                   int code4, const QbTables* __restrict__ tab)
{
    const int64_t bx = blockIdx.x;
    int i = 0;
    while (i + 1 < grp.count && bx >= grp.tile0[i + 1]) ++i;   // uniform: the kernel arguments are scalar
    const MmWeight& w = grp.w[i];
    mm_tile<XDT, DQ, MT, KF, XS>(x, M, K, w.codes, w.absmax, w.c2, w.absmax2, w.offset, log2B, log2B2, code4, w.N,
                                 w.y, tab, bx - grp.tile0[i]);
}

// ---------------------------------------------------------------------------
// many rows of activations: an LDS-tiled product
// ---------------------------------------------------------------------------
//
// For M above the small-batch regime the activations are worth sharing: one
// workgroup computes a tile of (16 TM) rows x (64 TN) columns of y.  Each
// step of 128 KH k stages the activation tile (16 TM rows x 128 KH k) in LDS,
// double-buffered, by direct global-to-LDS loads (no staging registers, no
// LDS store instructions).  The workgroup has 4 KH waves: wave w takes the columns
// 16 TN (w % 4) .. 16 TN (w % 4) + 16 TN - 1 and the k half w / 4 of every
// step (KH = 2), so every wave dequantizes only its own weights, once per
// workgroup, in registers, straight into MFMA B operands (W never passes
// through LDS).  With KH = 2 each SIMD holds two waves of the workgroup, and
// one wave's dequantization overlaps the other's products; their two partial
// sums meet in LDS at the end.  Per step a wave issues TM x TN x 4 MFMAs
// (16x16x32, compute dtype bf16 or fp16) against 32 weights per lane and
// column tile; the next step's activations and codes load meanwhile; one
// barrier per step.  Lanes use the k order of the small-M kernel within each
// 128 k (lane group g takes the 32 consecutive k at 32 g, MFMA q their k
// 8 q .. 8 q + 7), the same for both operands, so the sum is the same set of
// exact products.
// Requirements: K a multiple of 128 KH; 16-bit compute dtype.

constexpr int kGmStepK = 128;                      // k per wave and step


typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

template <int XDT, bool DQ, int TM, int TN, int KH>
__global__ __launch_bounds__(256 * KH) void k_dq4_gemm(const void* __restrict__ x, int64_t M, int64_t K,
                                                       const uint8_t* __restrict__ codes,
                                                       const float* __restrict__ absmax,
                                                       const uint8_t* __restrict__ c2,
                                                       const float* __restrict__ absmax2,
                                                       const float* __restrict__ offset, int log2B, int log2B2,
                                                       int code4, int64_t N, void* __restrict__ y,
                                                       const QbTables* __restrict__ tab)
{
    static_assert(XDT != DT_F32, "16-bit compute dtypes only");
    constexpr int NT = 256 * KH;                      // threads
    constexpr int BM = 16 * TM;                       // rows of the tile
    constexpr int BN = 64 * TN;                       // columns of the tile (4 wave columns x 16 TN)
    constexpr int SK = kGmStepK * KH;                 // k per workgroup step
    constexpr int PITCH = SK * 2;                     // bytes per LDS row of activations
    constexpr int RC = SK * 2 / 16;                   // 16-byte chunks per activation row and step
    constexpr int A_PER = BM * RC / NT;
    constexpr int NW = NT / 64;
    static_assert(A_PER * NT == BM * RC, "whole chunks per thread");
    static_assert(KH == 1 || 4 * TM * TN * 4 * 64 * 4 <= 2 * BM * PITCH, "partial sums fit the LDS tiles");
    __shared__ __attribute__((aligned(16))) char s_a[2 * BM * PITCH];
    __shared__ float s_val[16];
    __shared__ float s_dyn[DQ ? 256 : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wc = wave & 3, h = wave >> 2;           // column quarter, k half
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * BN, m0 = (int64_t)blockIdx.y * BM;
    const int64_t steps = K / SK;

    // rows past M read row M - 1 (their outputs are never stored)
    const char* const x_base = static_cast<const char*>(x) + m0 * K * 2;
    // direct loads: the wave's i-th load fills LDS bytes 1024 (i NW + wave)
    // onwards, 16 per lane; LDS chunk p of row R holds chunk p ^ (R % 16) of
    // the row (so the 16 rows of an MFMA operand read 16 different banks)
    uint32_t a_goff[A_PER], a_soff[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int o = (i * NW + wave) * 1024 + 16 * lane, row = o / PITCH, col = (o % PITCH) / 16 ^ (row & 15);
        const int grow = m0 + row < M ? row : (int)(M - 1 - m0);
        a_goff[i] = (uint32_t)(grow * K * 2 + col * 16);
        a_soff[i] = (uint32_t)((i * NW + wave) * 1024);
    }
    // weight rows of this lane: column tile j covers rows n0 + 16 (TN wc + j) + r;
    // the lane's 32 weights of a step start at k 128 h + 32 g
    const uint8_t* const cw_base = codes + n0 * K / 2;
    uint32_t cw_off[TN];
    int64_t e_row[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int64_t nr = 16 * (TN * wc + j) + r;
        const int64_t rn = n0 + nr < N ? nr : N - 1 - n0;
        cw_off[j] = (uint32_t)(rn * K / 2 + 64 * h + 16 * g);
        e_row[j] = (n0 + rn) * K + 128 * h + 32 * g;   // flat index of the lane's first weight of step 0
    }

    // codes and block constants: those of the step being computed (cw, sc,
    // sa) and of the next step, loading meanwhile (cwn, scn, san)
    u32x4 cw[TN], cwn[TN];
    uint32_t sc[TN], scn[TN];
    float sa[TN], san[TN];
    auto load_step = [&](int64_t s) {
        const char* const xs = x_base + s * SK * 2;
        char* const dst = s_a + (int)(s & 1) * BM * PITCH;
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            __builtin_amdgcn_global_load_lds((gptr_t)(xs + a_goff[i]), (lptr_t)(dst + a_soff[i]), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            cwn[j] = ldo<u32x4>(cw_base + s * (SK / 2), cw_off[j]);
            const int64_t blk = (e_row[j] + s * SK) >> log2B;
            if constexpr (DQ) {
                scn[j] = gld<uint8_t>(c2 + blk);
                san[j] = gld<float>(absmax2 + (blk >> log2B2));
            } else {
                san[j] = gld<float>(absmax + blk);
            }
        }
    };
    // the next step's data has landed (this wave's direct loads included)
    // and becomes the current one
    auto next_step = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            cw[j] = cwn[j];
            sc[j] = DQ ? scn[j] : 0u;
            sa[j] = san[j];
        }
    };

    load_step(0);
    if (tid < 16) s_val[tid] = (code4 == 0 ? tab->nf4 : tab->fp4)[tid];
    if constexpr (DQ) {
        if (tid < 256) s_dyn[tid] = tab->dyn8[tid];
    }
    const float mu = DQ ? gld<float>(offset) : 0.0f;
    next_step();
    __syncthreads();

    f32x4 acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[t][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    Frag<XDT> b[TN][4];
    auto dequant = [&]() {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const float a = DQ ? s_dyn[sc[j]] * sa[j] + mu : sa[j];   // two rounded operations (nested)
            dequant_chunk<XDT>(cw[j], a, s_val, b[j]);
        }
    };
    auto products = [&](int buf) {
        const char* const at = s_a + buf * BM * PITCH + r * PITCH;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                Frag<XDT> af;
                const int c = 16 * h + 4 * g + q;         // logical 16-byte chunk of the row
                const u32x4 v = *reinterpret_cast<const u32x4*>(at + t * 16 * PITCH + 16 * (c ^ r));
                af.w[0] = v.x;
                af.w[1] = v.y;
                af.w[2] = v.z;
                af.w[3] = v.w;
#pragma unroll
                for (int j = 0; j < TN; ++j) mma<XDT>(af, b[j][q], acc[t][j]);
            }
    };
    for (int64_t s = 0; s < steps; ++s) {
        const bool more = s + 1 < steps;
        dequant();
        if (more) load_step(s + 1);
        products((int)(s & 1));
        if (more) next_step();
        __syncthreads();
    }

    if constexpr (KH == 2) {
        // the k half 1 partial sums through LDS (free after the last barrier)
        float* const red = reinterpret_cast<float*>(s_a) + wc * (TM * TN * 4 * 64) + lane;
        if (h == 1) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[((t * TN + j) * 4 + i) * 64] = acc[t][j][i];
        }
        __syncthreads();
        if (h == 1) return;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[t][j][i] += red[((t * TN + j) * 4 + i) * 64];
    }

    // C of a 16x16 tile: lane (row / 4) * 16 + column, element row % 4
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t nn = n0 + 16 * (TN * wc + j) + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = m0 + 16 * t + 4 * g + i;
                if (m < M && nn < N) store1<XDT>(y, m * N + nn, acc[t][j][i]);
            }
        }
}

// Enqueue `kernel` on a 2-D grid of kMmThreads-thread workgroups; returns
// this launch's own status.
template <typename... KArgs, typename... Args>
hipError_t launch_2d_lds(void (*kernel)(KArgs...), dim3 grid, size_t lds, hipStream_t s, Args&&... args)
{
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kMmThreads), ptrs, lds, s);
        },
        vals);
}

template <typename... KArgs, typename... Args>
hipError_t launch_2d(void (*kernel)(KArgs...), dim3 grid, hipStream_t s, Args&&... args)
{
    return launch_2d_lds(kernel, grid, 0, s, std::forward<Args>(args)...);
}

// LDS bytes of M staged rows of K activations (whole steps, padded rows).
size_t xs_bytes(int64_t M, int64_t K)
{
    return (size_t)M * (size_t)(((K + kMmStepK - 1) / kMmStepK) * (kMmStepK / 8) + kXsPad) * 16;
}

template <int XDT, bool DQ, int MT, int XS = 0>
hipError_t mm_as(const void* x, int64_t M, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    const int64_t gx = (N + 15) / 16, gy = (M + 16 * MT - 1) / (16 * MT);
    if (gx >= (int64_t(1) << 31) || gy > 65535) return hipErrorInvalidValue;
    const size_t lds = XS ? xs_bytes(M, K) : 0;
    if (K % kMmStepK == 0)
        return launch_2d_lds(k_dq4_matmul<XDT, DQ, MT, true, XS>, dim3((unsigned)gx, (unsigned)gy), lds, s, x, M, K,
                             codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab);
    return launch_2d_lds(k_dq4_matmul<XDT, DQ, MT, false, XS>, dim3((unsigned)gx, (unsigned)gy), lds, s, x, M, K,
                         codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab);
}

// 16-bit activation rows that fit the LDS staging buffer: 0, else the
// prefetch depth in steps (1 while a wave has at most 4 steps of K).
template <int XDT>
int stage_x(int64_t M, int64_t K)
{
    if (XDT == DT_F32 || M < 1 || M > QB_MM_XS_ROWS) return 0;
    if (M * ((K + kMmStepK - 1) / kMmStepK) * kMmStepK * 2 > QB_MM_XS_BYTES) return 0;    // unpadded bytes
    const int64_t steps = (K + kMmStepK - 1) / kMmStepK;
    return (steps + kMmWaves - 1) / kMmWaves <= 4 ? 1 : 2;
}

// The tiled kernel on a grid of (BN-column, BM-row) tiles.
template <int XDT, bool DQ, int TM, int TN, int KH>
hipError_t gm_as(const void* x, int64_t M, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    const int64_t gx = (N + 64 * TN - 1) / (64 * TN), gy = (M + 16 * TM - 1) / (16 * TM);
    if (gx >= (int64_t(1) << 31) || gy > 65535) return hipErrorInvalidValue;
    std::tuple<const void*, int64_t, int64_t, const uint8_t*, const float*, const uint8_t*, const float*,
               const float*, int, int, int, int64_t, void*, const QbTables*>
        vals(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(k_dq4_gemm<XDT, DQ, TM, TN, KH>),
                                   dim3((unsigned)gx, (unsigned)gy), dim3(256 * KH), ptrs, 0, s);
        },
        vals);
}

// Rows of activations from which the tiled kernel takes over (16-bit compute
// dtypes, K a multiple of 128), and from which it uses the big tile shape.
#ifndef QB_GM_MIN_M
#define QB_GM_MIN_M 65
#endif
#ifndef QB_GM_BIG_M
#define QB_GM_BIG_M 512
#endif
// tile shapes (16 TM rows x 64 TN columns) below and from QB_GM_BIG_M rows
#ifndef QB_GM_SMALL_TM
#define QB_GM_SMALL_TM 4
#endif
#ifndef QB_GM_SMALL_TN
#define QB_GM_SMALL_TN 1
#endif
#ifndef QB_GM_BIG_TM
#define QB_GM_BIG_TM 8
#endif
#ifndef QB_GM_BIG_TN
#define QB_GM_BIG_TN 2
#endif

template <int XDT, bool DQ, int KH>
hipError_t gm_kh(int64_t M, const void* x, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    if (M >= QB_GM_BIG_M)
        return gm_as<XDT, DQ, QB_GM_BIG_TM, QB_GM_BIG_TN, KH>(x, M, K, codes, absmax, c2, absmax2, offset, log2B,
                                                              log2B2, code4, N, y, tab, s);
    return gm_as<XDT, DQ, QB_GM_SMALL_TM, QB_GM_SMALL_TN, KH>(x, M, K, codes, absmax, c2, absmax2, offset, log2B,
                                                              log2B2, code4, N, y, tab, s);
}

template <int XDT, bool DQ>
hipError_t mm_mt(int64_t M, const void* x, int64_t K, const uint8_t* codes, const float* absmax, const uint8_t* c2,
                 const float* absmax2, const float* offset, int log2B, int log2B2, int code4, int64_t N, void* y,
                 const QbTables* tab, hipStream_t s)
{
    if constexpr (XDT != DT_F32) {
        if (M >= QB_GM_MIN_M && K % (2 * kGmStepK) == 0)
            return gm_kh<XDT, DQ, 2>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
        if (M >= QB_GM_MIN_M && K % kGmStepK == 0)
            return gm_kh<XDT, DQ, 1>(M, x, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab, s);
    }
    if constexpr (XDT != DT_F32) {
        switch (stage_x<XDT>(M, K)) {
        case 1:
            return mm_as<XDT, DQ, 1, 1>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab,
                                        s);
        case 2:
            return mm_as<XDT, DQ, 1, 2>(x, M, K, codes, absmax, c2, absmax2, offset, log2B, log2B2, code4, N, y, tab,
                                        s);
        default: break;
        }
    }
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

namespace {

template <int XDT, bool DQ, int MT, int XS = 0>
hipError_t mmg_as(const void* x, int64_t M, int64_t K, const MmGroup& grp, int log2B, int log2B2, int code4,
                  const QbTables* tab, hipStream_t s)
{
    const int64_t gx = grp.tile0[grp.count], gy = (M + 16 * MT - 1) / (16 * MT);
    if (gx >= (int64_t(1) << 31) || gy > 65535) return hipErrorInvalidValue;
    const size_t lds = XS ? xs_bytes(M, K) : 0;
    if (K % kMmStepK == 0)
        return launch_2d_lds(k_dq4_matmul_grouped<XDT, DQ, MT, true, XS>, dim3((unsigned)gx, (unsigned)gy), lds, s, x,
                             M, K, grp, log2B, log2B2, code4, tab);
    return launch_2d_lds(k_dq4_matmul_grouped<XDT, DQ, MT, false, XS>, dim3((unsigned)gx, (unsigned)gy), lds, s, x,
                         M, K, grp, log2B, log2B2, code4, tab);
}

template <int XDT, bool DQ>
hipError_t mmg_mt(int64_t M, const void* x, int64_t K, const MmGroup& grp, int log2B, int log2B2, int code4,
                  const QbTables* tab, hipStream_t s)
{
    if constexpr (XDT != DT_F32) {
        switch (stage_x<XDT>(M, K)) {
        case 1: return mmg_as<XDT, DQ, 1, 1>(x, M, K, grp, log2B, log2B2, code4, tab, s);
        case 2: return mmg_as<XDT, DQ, 1, 2>(x, M, K, grp, log2B, log2B2, code4, tab, s);
        default: break;
        }
    }
    if (M <= 16) return mmg_as<XDT, DQ, 1>(x, M, K, grp, log2B, log2B2, code4, tab, s);
    if (M <= 32) return mmg_as<XDT, DQ, 2>(x, M, K, grp, log2B, log2B2, code4, tab, s);
    return mmg_as<XDT, DQ, 4>(x, M, K, grp, log2B, log2B2, code4, tab, s);
}

}  // namespace

hipError_t launch_dq4_matmul_grouped(const void* x, int xdt, int64_t M, int64_t K, const MmWeight* w, int count,
                                     int B, int B2, int code4, hipStream_t s)
{
    const bool dq = count > 0 && w[0].c2 != nullptr;
    // the tiled kernel's regime: one launch per weight (each has tiles enough)
    if (xdt != DT_F32 && M >= QB_GM_MIN_M && K % kGmStepK == 0) {
        for (int i = 0; i < count; ++i) {
            const hipError_t e = launch_dq4_matmul(x, xdt, M, K, w[i].codes, w[i].absmax, w[i].c2, w[i].absmax2,
                                                   w[i].offset, B, B2, code4, w[i].N, w[i].y, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (count < 1 || count > kMmGroupMax) return hipErrorInvalidValue;
    MmGroup grp{};
    grp.count = count;
    for (int i = 0; i < count; ++i) {
        grp.w[i] = w[i];
        grp.tile0[i + 1] = grp.tile0[i] + (w[i].N + 15) / 16;
    }
    for (int i = count; i < kMmGroupMax; ++i) grp.tile0[i + 1] = grp.tile0[count];
    int log2B = 0, log2B2 = 0;
    while ((1 << log2B) < B) ++log2B;
    while ((1 << log2B2) < B2) ++log2B2;
    switch (xdt) {
    case DT_BF16:
        return dq ? mmg_mt<DT_BF16, true>(M, x, K, grp, log2B, log2B2, code4, tab, s)
                  : mmg_mt<DT_BF16, false>(M, x, K, grp, log2B, log2B2, code4, tab, s);
    case DT_F16:
        return dq ? mmg_mt<DT_F16, true>(M, x, K, grp, log2B, log2B2, code4, tab, s)
                  : mmg_mt<DT_F16, false>(M, x, K, grp, log2B, log2B2, code4, tab, s);
    case DT_F32:
        return dq ? mmg_mt<DT_F32, true>(M, x, K, grp, log2B, log2B2, code4, tab, s)
                  : mmg_mt<DT_F32, false>(M, x, K, grp, log2B, log2B2, code4, tab, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qb
