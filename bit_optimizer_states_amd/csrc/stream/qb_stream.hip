// qb_stream.hip -- HBM reference streams for the benchmark (libqb_stream.so).
//
// Not part of the method: three plain streaming kernels that bound what any
// kernel of libqb can reach on the same device, in the same process, with the
// same access style (one 256-thread workgroup per 4096 floats, 16-byte
// non-temporal loads and stores, tiles in address order):
//   qbs_copy   dst[i] = src[i]        (n floats read, n written)
//   qbs_read   reads src[i]           (n floats read; nothing is written
//                                      unless the sum of a workgroup's values
//                                      is exactly `never`, which the caller
//                                      picks so that it does not happen)
//   qbs_write  dst[i] = value         (n floats written)
// n must be a multiple of 4096; pointers 16-byte aligned.  Asynchronous on
// `stream`; return 0 on success, else the HIP error code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
#define QBS_G __attribute__((address_space(1)))
constexpr int kPerWg = 1024;   // float4 per workgroup: 4 per thread

__global__ __launch_bounds__(256) void k_copy(const f4* __restrict__ src, f4* __restrict__ dst)
{
    const int64_t base = (int64_t)blockIdx.x * kPerWg + threadIdx.x;
    f4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load((const QBS_G f4*)(src + base + k * 256));
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v[k], (QBS_G f4*)(dst + base + k * 256));
}

__global__ __launch_bounds__(256) void k_read(const f4* __restrict__ src, float never, float* __restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * kPerWg + threadIdx.x;
    f4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 4; ++k) s += __builtin_nontemporal_load((const QBS_G f4*)(src + base + k * 256));
    const float t = (s.x + s.y) + (s.z + s.w);
    if (t == never) sink[threadIdx.x] = t;
}

__global__ __launch_bounds__(256) void k_write(f4* __restrict__ dst, float value)
{
    const int64_t base = (int64_t)blockIdx.x * kPerWg + threadIdx.x;
    const f4 v = {value, value, value, value};
#pragma unroll
    for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(v, (QBS_G f4*)(dst + base + k * 256));
}

int grid_of(int64_t n)
{
    if (n <= 0 || n % (4 * kPerWg) != 0 || n / (4 * kPerWg) >= (int64_t(1) << 31)) return -1;
    return (int)(n / (4 * kPerWg));
}

}  // namespace

extern "C" {

int qbs_copy(const float* src, float* dst, int64_t n, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !src || !dst) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const f4*>(src), reinterpret_cast<f4*>(dst));
    return (int)hipGetLastError();
}

int qbs_read(const float* src, int64_t n, float never, float* sink /* 256 floats */, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !src || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const f4*>(src), never, sink);
    return (int)hipGetLastError();
}

int qbs_write(float* dst, int64_t n, float value, void* stream)
{
    const int grid = grid_of(n);
    if (grid < 0 || !dst) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_write, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<f4*>(dst), value);
    return (int)hipGetLastError();
}

}  // extern "C"
