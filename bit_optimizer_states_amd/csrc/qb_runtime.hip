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

// Scratch of the allocation-free multi-tensor step: a device variable, so
// every device holds its own copy until the process ends.  Host code must not
// use the symbol's name as an address; device_scratch() returns the current
// device's copy, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* device_scratch()
{
    static std::mutex mu;
    static std::map<int, void*> by_device;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    auto it = by_device.find(dev);
    if (it != by_device.end()) return it->second;
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    by_device[dev] = ptr;
    return ptr;
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

size_t lds_for_wgs_per_cu(const void* kernel, int wgs)
{
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, size_t> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || wgs < 1) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    size_t dyn = 0;
    int per_cu = 0;
    hipFuncAttributes attr{};
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
        hipFuncGetAttributes(&attr, kernel) == hipSuccess && per_cu > 0) {
        const size_t share = (size_t)per_cu / (size_t)wgs;
        const size_t target = share > 512 ? share - 512 : 0;
        dyn = target > attr.sharedSizeBytes ? target - attr.sharedSizeBytes : 0;
    }
    cache[key] = dyn;
    return dyn;
}

__global__ __launch_bounds__(256) void k_clear_bins(unsigned long long* __restrict__ bins, int64_t nwords)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * 256) bins[i] = 0ull;
}

hipError_t launch_clear_bins(unsigned long long* bins, int sets, hipStream_t s)
{
    const int64_t nwords = (int64_t)sets * (int64_t)kBinWords;
    const int64_t grid = (nwords + 1023) / 1024;
    return launch_kernel(k_clear_bins, (int)(grid < 1024 ? grid : 1024), s, bins, nwords);
}

}  // namespace qb
