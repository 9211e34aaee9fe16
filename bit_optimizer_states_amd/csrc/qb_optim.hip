// qb_optim.hip -- the launches of the fused 8-bit optimizer steps (kernels in
// qb_optim_kernels.h; here the instantiations with every state in the signed
// dynamic code, the layer-wise kinds' second norm pass, and the launch entry
// points that pick them or the unsigned-code ones of qb_optim_uv.hip).
#include "qb_optim_kernels.h"

namespace qb {

// Layer-wise kinds, second pass: workgroup i adds the partial sums of tensor
// i's groups (thread t: groups t, t + 256, ... in order; then the butterfly
// and the waves in order), takes the norms and the ratio in binary64 and writes
// trust[i] = (float)(lr * ratio); a zero norm makes the ratio 1.
__global__ __launch_bounds__(256) void k_trust_scalars(TileMap<TensorDesc> gmap, const double* __restrict__ part,
                                                       int lamb, double lr, double wd, double eta,
                                                       float* __restrict__ trust)
{
    __shared__ double s_red[2][4];
    const int i = blockIdx.x, tid = threadIdx.x;
    const int64_t t0 = gmap.tile_begin[i], t1 = gmap.tile_begin[i + 1];
    double a = 0.0, b = 0.0;
    for (int64_t t = t0 + tid; t < t1; t += 256) {
        a += part[2 * t];
        b += part[2 * t + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
    }
    if ((tid & 63) == 0) {
        s_red[0][tid >> 6] = a;
        s_red[1][tid >> 6] = b;
    }
    __syncthreads();
    if (tid == 0) {
        const double sp = ((s_red[0][0] + s_red[0][1]) + s_red[0][2]) + s_red[0][3];
        const double sq = ((s_red[1][0] + s_red[1][1]) + s_red[1][2]) + s_red[1][3];
        const double pn = __builtin_sqrt(sp), qn = __builtin_sqrt(sq);
        double ratio = 1.0;
        if (pn > 0.0 && qn > 0.0) ratio = lamb ? pn / qn : (eta * pn) / (qn + wd * pn);
        trust[i] = (float)(lr * ratio);
    }
}

int64_t adamw_tiles(int64_t n, int B)
{
    const int64_t elems = (int64_t)kAdamThreads * (B >= 4 * kAdamThreads ? B / kAdamThreads : 4);
    return (n + elems - 1) / elems;
}

using namespace optim_dispatch;

hipError_t launch_optim8(int opt, const TensorDesc& single, const TileMap<TensorDesc>* map, int64_t ntiles, int B,
                         int pdt, int gdt, const OptScalars& hs, const float* trust, bool uv, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (opt_layerwise(opt) && !trust) return hipErrorInvalidValue;
    const OptLaunch a{&single, map, ntiles, &hs, tab, trust, nullptr, pdt, s};
    return uv ? optim_kind_uv(opt, B, gdt, a) : optim_kind<false>(opt, B, gdt, a);
}

hipError_t launch_trust_norms(int opt, const TileMap<TensorDesc>& gmap, int64_t ngroups, int B, int pdt, int gdt,
                              const OptScalars& hs, double* part, bool uv, hipStream_t s)
{
    const QbTables* tab = device_tables();
    if (!tab) return hipErrorNotInitialized;
    if (!opt_layerwise(opt) || !part) return hipErrorInvalidValue;
    const TensorDesc none{};
    const OptLaunch a{&none, &gmap, ngroups, &hs, tab, nullptr, part, pdt, s};
    return uv ? optim_kind_uv(opt, B, gdt, a) : optim_kind<false>(opt, B, gdt, a);
}

hipError_t launch_trust_scalars(int opt, const TileMap<TensorDesc>& gmap, const double* part, double lr,
                                double weight_decay, double trust_coefficient, float* trust, hipStream_t s)
{
    if (!opt_layerwise(opt) || gmap.count < 1) return hipErrorInvalidValue;
    return launch_kernel(k_trust_scalars, gmap.count, s, gmap, part, opt == OPT_LAMB ? 1 : 0, lr, weight_decay,
                         trust_coefficient, trust);
}

}  // namespace qb
