// Stand-ins for the device side of libqb (test infrastructure): the
// sanitizer build of the host code (qb_tables.cpp, qb_api.cpp) links these
// in place of the HIP sources.  No constant tables on any device, so every
// call that passes its checks stops with QB_EINIT before anything launches;
// a launcher reached anyway reports an error instead of running.
#include "qb_launch.h"

namespace qb {

const QbTables* device_tables() { return nullptr; }
void* device_scratch() { return nullptr; }

int64_t adamw_tiles(int64_t n, int B)
{
    const int64_t elems = 256 * (B >= 1024 ? B / 256 : 4);
    return (n + elems - 1) / elems;
}

hipError_t launch_clear_bins(unsigned long long*, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quant(const QuantDesc&, const TileMap<QuantDesc>*, int64_t, int, int, int, int, bool,
                        unsigned long long*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_quant_user(const QuantDesc&, int64_t, int, int, const UserCode*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_dequant_user(const DequantDesc&, int64_t, int, int, const UserCode*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_normalize(const void*, int, int64_t, const float*, int64_t, float*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_chunk_quantiles(const void*, int, int64_t, float*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quantile_code(const float*, int64_t, double*, double*, UserCode*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_dq4_matmul(const void*, int, int64_t, int64_t, const uint8_t*, const float*, const uint8_t*,
                             const float*, const float*, int, int, int, int64_t, void*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_dq4_matmul_grouped(const void*, int, int64_t, int64_t, const MmWeight*, int, int, int, int,
                                     hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_dq_mean(const QuantDesc&, const TileMap<QuantDesc>*, int, const unsigned long long*, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_dequant(const DequantDesc&, const TileMap<DequantDesc>*, int64_t, int, int, int, int, bool, int,
                          hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_optim8(int, const TensorDesc&, const TileMap<TensorDesc>*, int64_t, int, int, int,
                         const OptScalars&, const float*, bool, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_trust_norms(int, const TileMap<TensorDesc>&, int64_t, int, int, int, const OptScalars&, double*,
                              bool, hipStream_t)
{
    return hipErrorInvalidValue;
}
hipError_t launch_trust_scalars(int, const TileMap<TensorDesc>&, const double*, double, double, double, float*,
                                hipStream_t)
{
    return hipErrorInvalidValue;
}

}  // namespace qb
