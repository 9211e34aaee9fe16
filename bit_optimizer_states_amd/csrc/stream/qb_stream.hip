// qb_stream.hip -- HBM reference streams for the benchmark (libqb_stream.so).
//
// Not part of the method: three plain streaming kernels that bound what any
// kernel of libqb can reach on the same device and in the same process.  They
// take the fastest plain form measured on MI355X: one 16-byte non-temporal
// access per thread, one 256-thread workgroup per 1024 floats, and the tiles
// dealt out so that each XCD walks its own contiguous eighth of the buffer
// (copy 6.6-6.7 TB/s on 4 GiB; four accesses per thread in address order
// reached 5.6-5.7):
//   qbs_copy   dst[i] = src[i]        (n floats read, n written)
//   qbs_read   reads src[i]           (n floats read; nothing is written
//                                      unless the sum of a thread's 4 values
//                                      is exactly `never`, which the caller
//                                      picks so that it does not happen)
//   qbs_write  dst[i] = value         (n floats written)
// n must be a positive multiple of 1024; pointers 16-byte aligned.
// Asynchronous on `stream`; return 0 on success, else the HIP error code.
//
// Two more streams repeat the exact memory accesses of libqb's two headline
// kernels on the caller's own buffers, with no arithmetic: what those access
// patterns reach on the same physical pages.
//   qbs_adamw_pattern    the multi-tensor 8-bit AdamW step (fp32 p, bf16 g,
//                        8-bit m and v, block 2048): every tensor's bytes are
//                        read and written back unchanged (g only read)
//   qbs_dequant4_pattern the grouped nested 4-bit dequantize to bf16 (block
//                        64, second level 256): codes, nested codes and
//                        second-level absmax read, y written (its values are
//                        not a dequantization)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

// One tensor of the access-pattern streams (see qb_stream.h).
struct QbsAdamTensor {
    float* p;
    const uint16_t* g;
    uint8_t* m;
    uint8_t* v;
    float* am;
    float* av;
    int64_t n;
    int64_t pad;
};
struct QbsDequantTensor {
    const uint8_t* codes;
    const uint8_t* c2;
    const float* absmax2;
    const float* offset;
    uint16_t* y;
    int64_t n;
    int64_t pad[2];
};
#define QBS_G __attribute__((address_space(1)))
constexpr int kThreads = 256;   // one float4 per thread
constexpr int kXcds = 8;

// Workgroup b runs on XCD b % 8 (round-robin dispatch); give XCD x the x-th
// contiguous range of tiles, in order.
__device__ __forceinline__ int64_t tile_of(int64_t b, int64_t ntiles)
{
    const int64_t q = ntiles / kXcds, r = ntiles % kXcds, x = b % kXcds, k = b / kXcds;
    return x * q + (x < r ? x : r) + k;
}

__global__ __launch_bounds__(kThreads) void k_copy(const f4* __restrict__ src, f4* __restrict__ dst)
{
    const int64_t i = tile_of(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    __builtin_nontemporal_store(__builtin_nontemporal_load((const QBS_G f4*)(src + i)), (QBS_G f4*)(dst + i));
}

__global__ __launch_bounds__(kThreads) void k_read(const f4* __restrict__ src, float never, float* __restrict__ sink)
{
    const int64_t i = tile_of(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    const f4 s = __builtin_nontemporal_load((const QBS_G f4*)(src + i));
    const float t = (s.x + s.y) + (s.z + s.w);
    if (t == never) sink[threadIdx.x] = t;
}

__global__ __launch_bounds__(kThreads) void k_write(f4* __restrict__ dst, float value)
{
    const int64_t i = tile_of(blockIdx.x, gridDim.x) * kThreads + threadIdx.x;
    const f4 v = {value, value, value, value};
    __builtin_nontemporal_store(v, (QBS_G f4*)(dst + i));
}

// ---------------------------------------------------------------------------
// access patterns of the headline kernels (no arithmetic)
// ---------------------------------------------------------------------------

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ T ntl(const void* base, uint32_t off)
{
    return __builtin_nontemporal_load((const QBS_G T*)(static_cast<const char*>(base) + off));
}

template <class T>
__device__ __forceinline__ void nts(void* base, uint32_t off, T v)
{
    __builtin_nontemporal_store(v, (QBS_G T*)(static_cast<char*>(base) + off));
}

template <class T>
__device__ __forceinline__ T gl(const T* p)
{
    return *(const QBS_G T*)p;
}

template <class T>
__device__ __forceinline__ void gs(T* p, T v)
{
    *(QBS_G T*)p = v;
}

// The tensor holding global tile `tile` (tile_begin ascending, count + 1
// entries): binary search with uniform scalar loads.
__device__ __forceinline__ int tensor_of(const int64_t* __restrict__ tile_begin, int count, int64_t tile)
{
    int lo = 0, hi = count;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_begin[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// A value the compiler must treat as changed (no instruction).
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ float opaque(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ f4 opaque(f4 v)
{
    return f4{opaque(v.x), opaque(v.y), opaque(v.z), opaque(v.w)};
}

constexpr int kAdamBlock = 2048;   // one 256-thread workgroup per block, 8 elements per thread

__global__ __launch_bounds__(kThreads) void k_adamw_pattern(const QbsAdamTensor* __restrict__ t,
                                                            const int64_t* __restrict__ tile_begin, int count)
{
    const int64_t tile = tile_of(blockIdx.x, gridDim.x);
    const int ti = tensor_of(tile_begin, count, tile);
    const QbsAdamTensor d = t[ti];
    const int64_t lt = tile - tile_begin[ti];
    const int tid = threadIdx.x;
    const int64_t tbase = lt * kAdamBlock;
    const int64_t rem = d.n - tbase;
    char* const pt = reinterpret_cast<char*>(d.p) + tbase * 4;
    const char* const gt = reinterpret_cast<const char*>(d.g) + tbase * 2;
    uint8_t* const mt = d.m + tbase;
    uint8_t* const vt = d.v + tbase;
    float am = opaque(gl(d.am + lt)), av = opaque(gl(d.av + lt));
    if (rem >= kAdamBlock) {
        f4 p[2];
        u2 g[2];
        uint32_t m[2], v[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t e = (uint32_t)(tid * 4 + c * 1024);
            p[c] = ntl<f4>(pt, e * 4);
            g[c] = ntl<u2>(gt, e * 2);
            m[c] = ntl<uint32_t>(mt, e);
            v[c] = ntl<uint32_t>(vt, e);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            asm volatile("" ::"v"(g[c].x), "v"(g[c].y));
            const uint32_t e = (uint32_t)(tid * 4 + c * 1024);
            nts<f4>(pt, e * 4, opaque(p[c]));
            nts<uint32_t>(mt, e, opaque(m[c]));
            nts<uint32_t>(vt, e, opaque(v[c]));
        }
    } else {
#pragma unroll 1
        for (int c = 0; c < 2; ++c)
#pragma unroll 1
            for (int j = 0; j < 4; ++j) {
                const int64_t e = tid * 4 + c * 1024 + j;
                if (e < rem) {
                    float* const pe = reinterpret_cast<float*>(pt) + e;
                    gs(pe, opaque(gl(pe)));
                    asm volatile("" ::"v"((uint32_t)gl(reinterpret_cast<const uint16_t*>(gt) + e)));
                    gs(mt + e, (uint8_t)opaque((uint32_t)gl(mt + e)));
                    gs(vt + e, (uint8_t)opaque((uint32_t)gl(vt + e)));
                }
            }
    }
    if (tid == 0) {
        gs(d.am + lt, am);
        gs(d.av + lt, av);
    }
}

constexpr int kDqTile = 8192;      // one 256-thread workgroup per 8192 weights, 4 units of 8 per thread

__global__ __launch_bounds__(kThreads) void k_dequant4_pattern(const QbsDequantTensor* __restrict__ t,
                                                               const int64_t* __restrict__ tile_begin, int count)
{
    const int64_t tile = tile_of(blockIdx.x, gridDim.x);
    const int ti = tensor_of(tile_begin, count, tile);
    const QbsDequantTensor d = t[ti];
    const int64_t lt = tile - tile_begin[ti];
    const int tid = threadIdx.x;
    const int64_t tbase = lt * kDqTile;
    const int64_t rem = d.n - tbase;
    const uint8_t* const ct = d.codes + tbase / 2;
    char* const yt = reinterpret_cast<char*>(d.y) + tbase * 2;
    // block constants: one 64-weight block per thread (128 per tile)
    const int64_t blk = tbase / 64 + tid;
    uint32_t sc = 0;
    if (tid < kDqTile / 64 && blk * 64 < d.n) {
        sc = gl(d.c2 + blk);
        sc ^= __float_as_uint(gl(d.absmax2 + (blk >> 8)));
    }
    sc ^= __float_as_uint(gl(d.offset));
    asm volatile("" ::"v"(sc));
    if (rem >= kDqTile) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = ntl<uint32_t>(ct, (uint32_t)(k * kThreads + tid) * 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = opaque(w[k]);
            nts<u4>(yt, (uint32_t)(k * kThreads + tid) * 16, u4{x, x, x, x});
        }
    } else {
#pragma unroll 1
        for (int k = 0; k < 4; ++k)
#pragma unroll 1
            for (int j = 0; j < 8; ++j) {
                const int64_t e = (int64_t)(k * kThreads + tid) * 8 + j;
                if (e < rem) gs(reinterpret_cast<uint16_t*>(yt) + e, (uint16_t)opaque((uint32_t)gl(ct + e / 2)));
            }
    }
}

int grid_of(int64_t n)
{
    if (n <= 0 || n % (4 * kThreads) != 0 || n / (4 * kThreads) >= (int64_t(1) << 31)) return -1;
    return (int)(n / (4 * kThreads));
}

}  // namespace

extern "C" {

int qbs_copy(const float* src, float* dst, int64_t n, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !src || !dst) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst));
    return (int)hipGetLastError();
}

int qbs_read(const float* src, int64_t n, float never, float* sink /* 256 floats */, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !src || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const f4*>(src), never, sink);
    return (int)hipGetLastError();
}

int qbs_write(float* dst, int64_t n, float value, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !dst) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_write, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<f4*>(dst), value);
    return (int)hipGetLastError();
}

// tensors, tile_begin: device arrays (count descriptors; count + 1 first
// tiles, the last the total = the grid)
int qbs_adamw_pattern(const void* tensors, const int64_t* tile_begin, int count, int64_t ntiles, void* stream)
{
    if (!tensors || !tile_begin || count < 1 || ntiles < 1 || ntiles >= (int64_t(1) << 31))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_adamw_pattern, dim3((unsigned)ntiles), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const QbsAdamTensor*>(tensors), tile_begin, count);
    return (int)hipGetLastError();
}

int qbs_dequant4_pattern(const void* tensors, const int64_t* tile_begin, int count, int64_t ntiles, void* stream)
{
    if (!tensors || !tile_begin || count < 1 || ntiles < 1 || ntiles >= (int64_t(1) << 31))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_dequant4_pattern, dim3((unsigned)ntiles), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const QbsDequantTensor*>(tensors), tile_begin,
                       count);
    return (int)hipGetLastError();
}

}  // extern "C"
