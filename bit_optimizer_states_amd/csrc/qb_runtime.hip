// qb_runtime.hip -- per-device constant tables, launch sizing, small kernels.
#include <map>
#include <mutex>
#include <utility>

#include "qb_device.h"
#include "qb_launch.h"

namespace qb {

// One copy of the tables per device, filled once from the host build.
__device__ QbTables g_tables;

const QbTables* device_tables()
{
    static std::mutex mu;
    static std::map<int, const QbTables*> by_device;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    auto it = by_device.find(dev);
    if (it != by_device.end()) return it->second;
    const QbTables* host = host_tables();
    if (!host) return nullptr;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_tables), host, sizeof(QbTables), 0, hipMemcpyHostToDevice) != hipSuccess)
        return nullptr;
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(g_tables)) != hipSuccess || !addr) return nullptr;
    by_device[dev] = static_cast<const QbTables*>(addr);
    return static_cast<const QbTables*>(addr);
}

int persistent_grid_cap(const void* kernel, int (*query)(const void*))
{
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1024;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    int cap = cus * query(kernel);
    cache[key] = cap;
    return cap;
}

__global__ __launch_bounds__(256) void k_clear_bins(unsigned long long* __restrict__ bins)
{
#pragma unroll
    for (int k = 0; k < kBinCopies; ++k) bins[k * 256 + threadIdx.x] = 0ull;
}

hipError_t launch_clear_bins(unsigned long long* bins, hipStream_t s)
{
    return launch_kernel(k_clear_bins, 1, s, bins);
}

}  // namespace qb
