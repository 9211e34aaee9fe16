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
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
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

}  // extern "C"
