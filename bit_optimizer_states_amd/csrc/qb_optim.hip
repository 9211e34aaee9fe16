// qb_optim.hip -- fused 8-bit optimizer steps: AdamW, Adam, Lion, SGD with
// momentum, RMSprop and the layer-wise LAMB and LARS, each state held as
// block-wise dynamic 8-bit codes.
//
// The 8-bit optimizer keeps its states as block-wise dynamic 8-bit codes plus
// one fp32 absmax per block (abstract quoted on "Py之bitsandbytes：
// bitsandbytes的简介、安装、使用方法之详细攻略", section 2; 2 bytes of state per
// parameter for Adam: "bitsandbytes - Quantização de LLM", section Workflow
// 3) and replaces its 32-bit optimizer with the same hyperparameters; 8-bit
// Adam, SGD, RMSprop and Lion are listed beside AdamW ("bitsandbytes深度解析",
// section 优化器模块深度分析).  One pass per block, in registers: decode the
// states, update them and p, reduce each state's new block absmax, encode the
// states again.  Each parameter's bytes cross HBM once.
//
// One 256-thread workgroup per tile (a tile is one block for B >= 1024), in
// tile order.  For many tensors, the tiles of all tensors are numbered in one
// range; a workgroup finds its tensor from a coarse bucket index (the tensor
// holding the bucket's first tile) and, only where a bucket spans several
// tensors, a binary search among those (uniform, scalar loads that stay in
// the scalar cache).  Parameters are binary32, or 16-bit (widened on load,
// rounded once to nearest even on store).  The layer-wise kinds LAMB and
// LARS need each tensor's norms before any parameter moves: a norm pass
// (k_trust_norms, k_trust_scalars) precedes their step.
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
