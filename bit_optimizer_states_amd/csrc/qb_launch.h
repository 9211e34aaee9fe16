// qb_launch.h -- internal launchers behind the C ABI (argument checks are done
// by the callers in qb_api.cpp; these only pick the kernel and enqueue it).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "qb_tables.h"

namespace qb {

// Exponent bins of the nested-quantization mean at the start of the workspace:
// kBinCopies copies of 256 uint64 words (254 used; workgroup w adds into copy
// w % kBinCopies: with 8 copies the device-scope atomics of the grouped 7B
// quantize queued on a few addresses, 3.22 ms against 2.90 ms with 64), then
// the fp32 absmax of the first level.
#ifndef QB_BIN_COPIES
#define QB_BIN_COPIES 64
#endif
constexpr int kBinCopies = QB_BIN_COPIES;
constexpr size_t kBinWords = (size_t)kBinCopies * 256;
constexpr size_t kBinBytes = kBinWords * sizeof(unsigned long long);

// Optimizer kinds of the fused 8-bit step (the values of qb_optimizer).
enum OptKind { OPT_ADAMW = 0, OPT_ADAM = 1, OPT_LION = 2, OPT_SGD = 3, OPT_RMSPROP = 4, OPT_LAMB = 5, OPT_LARS = 6 };
constexpr bool opt_layerwise(int opt) { return opt == OPT_LAMB || opt == OPT_LARS; }
constexpr int32_t kOptNesterov = 1, kOptFirstStep = 2;

// Host scalars of one step, each computed in binary64 and rounded once:
//   Adam(W)  b1, ob1 = 1 - b1, b2, ob2, s1 = lr / (1 - b1^t), s2 = 1 / sqrt(1 - b2^t),
//            dec = 1 - lr*wd (AdamW), eps, wd (Adam's L2 term);
//   Lion     b1, ob1, b2, ob2, lr, dec = 1 - lr*wd;
//   SGD      b1 = momentum, omd = 1 - dampening, lr, wd, flags;
//   RMSprop  b2 = alpha, ob2 = 1 - alpha, lr, eps, wd;
//   LAMB     Adam's b1 .. s2 with s1 = 1 / (1 - b1^t) (no lr), eps, wd;
//   LARS     b1 = momentum, wd.
// The layer-wise kinds take their per-tensor S = (float)(lr * ratio) from a
// device array in place of lr.
struct OptScalars {
    float b1, ob1, b2, ob2, s1, s2, dec, eps;
    float wd, lr, omd;
    int32_t flags;
};

// One tensor of a fused optimizer launch (p of the launch's parameter dtype);
// tile_begin is the first global tile.
struct TensorDesc {
    void* p;
    const void* g;
    uint8_t* m;
    uint8_t* v;
    float* am;
    float* av;
    int64_t n;
    int64_t tile_begin;
};
static_assert(sizeof(TensorDesc) == 64, "descriptor layout");

// A user code in device memory (qb_code_table_bytes() bytes): 256 ascending
// entries and their decision thresholds, thr[k] = the smallest binary32 that
// encodes to entry k+1 or above (thr[255] = +inf), so code = #{k : n >= thr[k]};
// then the index of the thresholds by bucket of n (user_bucket, first[]).
struct UserCode {
    float values[256];
    float thr[256];
    uint8_t first[kUserFirstBytes];
};
static_assert(sizeof(UserCode) == 6160, "user code layout");

// One tensor of a quantization pass; tile_begin is its first global tile.
// First pass: x [n] of the input dtype, codes out, absmax out (the caller's,
// or the fp32 workspace of a nested quantization).  Second pass of
// a nested quantization: x = that fp32 absmax [n = its count], codes = the
// nested codes, absmax = the second-level absmax, offset[0] = the mean.
struct QuantDesc {
    const void* x;
    uint8_t* codes;
    float* absmax;
    float* offset;
    int64_t n;
    int64_t tile_begin;
    int64_t pad[2];
};
static_assert(sizeof(QuantDesc) == 64, "descriptor layout");

// One tensor of a grouped dequantization; tile_begin is its first global tile.
struct DequantDesc {
    const uint8_t* codes;
    const float* absmax;      // per-block absmax (plain), or nullptr (nested)
    const uint8_t* c2;        // nested state: codes, second-level absmax, mean
    const float* absmax2;
    const float* offset;
    void* y;
    int64_t n;
    int64_t tile_begin;
};
static_assert(sizeof(DequantDesc) == 64, "descriptor layout");

// Device tables of a multi-tensor launch: `count` descriptors; the first tile
// of every tensor (count + 1 entries, the last one the total); and a coarse
// index, bucket_first[k] = the tensor that holds tile k << shift (one entry
// per bucket plus a last one = count - 1), so that a workgroup finds its tensor
// with two dependent loads instead of a binary search over all tensors.
template <class Desc>
struct TileMap {
    const Desc* descs;
    const int64_t* tile_begin;
    const int32_t* bucket_first;
    int32_t count;
    int32_t shift;
};

constexpr int64_t max_tile_buckets(int64_t count) { return 2 * count + 64; }

// Device copy of the constant tables for the current device (uploaded once).
const QbTables* device_tables();

// The library's own scratch for the allocation-free multi-tensor step: the
// tables of one multi-tensor launch (descriptors, first tiles, bucket index)
// of at most kScratchMaxTensors tensors.  device_scratch() is its address on
// the current device (nullptr on a HIP error).
constexpr int32_t kScratchMaxTensors = 4096;
constexpr size_t kScratchBytes = 384 * 1024;
static_assert((size_t)kScratchMaxTensors * 64 + ((size_t)kScratchMaxTensors + 1) * 8 +
                      ((size_t)max_tile_buckets(kScratchMaxTensors) + 1) * 4 <= kScratchBytes,
              "scratch holds the tables of kScratchMaxTensors tensors");
void* device_scratch();

// CUs x resident workgroups per CU of a kernel, cached per (device, kernel);
// `query` returns the kernel's resident workgroups per CU.
int persistent_grid_cap(const void* kernel, int (*query)(const void*));

// Dynamic LDS for `kernel` that brings a workgroup's LDS to a 1/wgs share of a
// CU's (less 512 bytes of allocation slack), so that at most `wgs` of its
// workgroups are resident on a CU at once; 0 where its own LDS already allows
// no more.  Cached per (device, kernel); 0 on a HIP error.
size_t lds_for_wgs_per_cu(const void* kernel, int wgs);

// Workgroups to launch for a persistent grid-stride kernel: enough to fill
// every CU at the kernel's occupancy, never more than there are tiles.
template <class Kernel>
int persistent_grid(Kernel kernel, int64_t ntiles)
{
    auto query = [](const void* k) -> int {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<Kernel>(const_cast<void*>(k)), 256, 0)
                != hipSuccess || per_cu < 1)
            per_cu = 1;
        return per_cu;
    };
    int cap = persistent_grid_cap(reinterpret_cast<const void*>(kernel), query);
    return (int)(ntiles < cap ? (ntiles > 0 ? ntiles : 1) : cap);
}

// Enqueue `kernel` with 256-thread workgroups; returns this launch's own
// status (a stale error of an earlier call is neither returned nor cleared).
template <typename... KArgs, typename... Args>
hipError_t launch_kernel_nt(void (*kernel)(KArgs...), int grid, int threads, hipStream_t s, Args&&... args)
{
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(threads), ptrs, 0, s);
        },
        vals);
}

// The same with `lds` bytes of dynamic LDS per workgroup.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel_lds(void (*kernel)(KArgs...), int grid, int threads, size_t lds, hipStream_t s,
                             Args&&... args)
{
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    return std::apply(
        [&](auto&... v) {
            void* ptrs[] = {static_cast<void*>(&v)...};
            return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(threads), ptrs, lds, s);
        },
        vals);
}

template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), int grid, hipStream_t s, Args&&... args)
{
    return launch_kernel_nt(kernel, grid, 256, s, std::forward<Args>(args)...);
}

// Zero `sets` sets of nested-quantization exponent bins (kBinWords each).
hipError_t launch_clear_bins(unsigned long long* bins, int sets, hipStream_t s);

// Elements per tile of the quantization kernel: QB_Q_TILE for 8-bit codes,
// QB_Q4_TILE for 4-bit codes, or one sub-tile of 256 threads x B / 256
// elements where that is larger (B = 4096).  Measured on MI355X (same box, 7B
// weights, codes bit for bit the same): 8192 against 4096 makes the 4-bit
// nested quantize 3.6-4.3% faster, the 8-bit quantize and dequantize of
// 268M values 7-10% slower; 16384 is slower than 8192 for both.
#ifndef QB_Q_TILE
#define QB_Q_TILE 4096
#endif
#ifndef QB_Q4_TILE
#define QB_Q4_TILE 8192
#endif
constexpr int64_t quant_tile_elems(int B, int bits)
{
    return B > (bits == 4 ? QB_Q4_TILE : QB_Q_TILE) ? B : (bits == 4 ? QB_Q4_TILE : QB_Q_TILE);
}

// Quantize one tensor (map == nullptr) or the tensors of `map` (ntiles in
// all); bits 8 (dynamic code) or 4 (code4: 0 NF4, 1 FP4).  bins: the exponent
// bins of a nested first pass (tensor i of the map uses set i), else nullptr.
// second: the nested second pass (bits 8, fp32 input, mean in offset[0]).
hipError_t launch_quant(const QuantDesc& single, const TileMap<QuantDesc>* map, int64_t ntiles, int bits, int code4,
                        int B, int xdt, bool second, unsigned long long* bins, hipStream_t s);

// Quantize / dequantize one tensor with a user code (8-bit codes).
hipError_t launch_quant_user(const QuantDesc& d, int64_t ntiles, int B, int xdt, const UserCode* code, hipStream_t s);
hipError_t launch_dequant_user(const DequantDesc& d, int64_t ntiles, int B, int ydt, const UserCode* code,
                               hipStream_t s);

// Quantile estimation: chunks of kQuantileChunk consecutive values, each
// sorted on its own; E holds 257 order statistics per chunk ([257][nchunks]),
// S the binary64 sums per group of 256 chunks ([257][ngroups]).
constexpr int kQuantileChunk = 4096;
hipError_t launch_normalize(const void* x, int xdt, int64_t n, const float* absmax, int64_t B, float* out,
                            hipStream_t s);
hipError_t launch_chunk_quantiles(const void* x, int xdt, int64_t n, float* E, hipStream_t s);
hipError_t launch_quantile_code(const float* E, int64_t nchunks, double* A, double* averages, UserCode* out,
                                hipStream_t s);

// y [M, N] = x [M, K] W^T in compute dtype xdt (fp32, fp16, bf16; y the same),
// W [N, K] as 4-bit codes (code4: 0 NF4, 1 FP4) with block size B and either
// absmax (plain) or c2 / absmax2 / offset (nested, block size B2).  K is a
// multiple of 32; x, codes and y are 16-byte aligned.
hipError_t launch_dq4_matmul(const void* x, int xdt, int64_t M, int64_t K, const uint8_t* codes, const float* absmax,
                             const uint8_t* c2, const float* absmax2, const float* offset, int B, int B2, int code4,
                             int64_t N, void* y, hipStream_t s);

// One weight of a grouped product: plain (absmax) or nested (c2, absmax2,
// offset); y [M, N].
struct MmWeight {
    const uint8_t* codes;
    const float* absmax;
    const uint8_t* c2;
    const float* absmax2;
    const float* offset;
    void* y;
    int64_t N;
};
constexpr int kMmGroupMax = 8;

// launch_dq4_matmul for `count` (1 .. kMmGroupMax) weights against the same x,
// all plain or all nested, one code and block sizes: one launch in the
// small-M regime, one launch per weight in the tiled kernel's.
hipError_t launch_dq4_matmul_grouped(const void* x, int xdt, int64_t M, int64_t K, const MmWeight* w, int count,
                                     int B, int B2, int code4, hipStream_t s);

// Exact mean of the absmax of one tensor (map == nullptr) or of the `count`
// tensors of map (second-pass descriptors) into offset[0].
hipError_t launch_dq_mean(const QuantDesc& single, const TileMap<QuantDesc>* map, int count,
                          const unsigned long long* bins, hipStream_t s);

// Dequantize one tensor (map == nullptr) or the tensors of `map` (ntiles in
// all); bits 8 (dynamic code) or 4 (code4: 0 NF4, 1 FP4); dq: nested absmax.
hipError_t launch_dequant(const DequantDesc& single, const TileMap<DequantDesc>* map, int64_t ntiles, int bits,
                          int code4, int B, int B2, bool dq, int ydt, hipStream_t s);

// Elements per tile of the dequantization kernel: 4-bit codes for one tensor
// and for a grouped launch, and 8-bit codes into binary32 and into 16-bit
// outputs.  Measured on MI355X: 8192, 8192 and 4096 are the best of 4096 /
// 8192 / 16384 (2048 takes the 4-bit sweep from 2.75 to 3.94 ms); 8-bit codes
// into binary32 run 12% faster in tiles of 2048 (0.213 against 0.238 ms on
// 268M values), i.e. 8 KB written per workgroup, as 4096 gives the 16-bit
// outputs (2048 there: 0.160 against 0.125 ms).
#ifndef QB_DQ_TILE
#define QB_DQ_TILE 8192
#endif
#ifndef QB_DQ_MULTI_TILE
#define QB_DQ_MULTI_TILE 8192
#endif
#ifndef QB_DQ8_TILE
#define QB_DQ8_TILE 4096
#endif
#ifndef QB_DQ8_F32_TILE
#define QB_DQ8_F32_TILE 2048
#endif
constexpr int64_t dequant_tile_elems(int bits, bool multi, int ydt)
{
    return bits == 8 ? (ydt == 0 ? QB_DQ8_F32_TILE : QB_DQ8_TILE) : (multi ? QB_DQ_MULTI_TILE : QB_DQ_TILE);
}
// Fused 8-bit step of optimizer `opt` (OptKind) on one tensor (map ==
// nullptr) or on the tensors of map.
// trust: the per-tensor step scalars S of the layer-wise kinds (indexed like
// map->descs), nullptr for the others.
// pdt: the parameters' dtype (binary32, or a 16-bit type equal to gdt).
// uv: the never-negative state (v of AdamW, Adam and LAMB; RMSprop's state)
// is held in the unsigned dynamic code (only those kinds).
hipError_t launch_optim8(int opt, const TensorDesc& single, const TileMap<TensorDesc>* map, int64_t ntiles, int B,
                         int pdt, int gdt, const OptScalars& hs, const float* trust, bool uv, hipStream_t s);

// Layer-wise kinds, before launch_optim8: per group of kNormGroupTiles
// consecutive optimizer tiles of one tensor (gmap: the tensors with
// tile_begin = their first group; ngroups in all), the partial sums of |p|^2
// and of |u|^2 (LAMB) or |g|^2 (LARS) in binary64 (part[2 * group],
// part[2 * group + 1]); then one workgroup per tensor adds its groups' partials
// in a fixed order and writes trust[tensor] = (float)(lr * ratio).
constexpr int64_t kNormGroupTiles = 32;
hipError_t launch_trust_norms(int opt, const TileMap<TensorDesc>& gmap, int64_t ngroups, int B, int pdt, int gdt,
                              const OptScalars& hs, double* part, bool uv, hipStream_t s);
hipError_t launch_trust_scalars(int opt, const TileMap<TensorDesc>& gmap, const double* part, double lr,
                                double weight_decay, double trust_coefficient, float* trust, hipStream_t s);

// Tiles of the optimizer kernel for a tensor of n elements at block size B.
int64_t adamw_tiles(int64_t n, int B);

}  // namespace qb
