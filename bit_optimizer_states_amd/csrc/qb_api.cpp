// qb_api.cpp -- the C ABI declared in include/qb.h: argument validation, host
// scalars, workspace layout and kernel dispatch.  Nothing is enqueued unless
// every argument checks out.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "qb.h"
#include "qb_launch.h"
#include "qb_tables.h"

namespace {

using namespace qb;

bool pow2_block(int32_t b) { return b >= 64 && b <= 4096 && (b & (b - 1)) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(qb_dtype d) { return d == QB_F32 || d == QB_F16 || d == QB_BF16; }
bool valid_code(qb_code c) { return c == QB_DYN8 || c == QB_NF4 || c == QB_FP4; }
bool is4(qb_code c) { return c == QB_NF4 || c == QB_FP4; }
int code4_index(qb_code c) { return c == QB_NF4 ? 0 : 1; }
int64_t nblocks(int64_t n, int32_t b) { return (n + b - 1) / b; }

qb_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return QB_OK;
    if (e == hipErrorNotInitialized) return QB_EINIT;
    return QB_EHIP;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks shared by quantize and dequantize for the nested state.
qb_status check_dq(const qb_dq* dq, int64_t nb, bool need_ws)
{
    if (!dq->codes || !dq->absmax2 || !dq->offset) return QB_EINVAL;
    if (!pow2_block(dq->blocksize2)) return QB_EINVAL;
    if (!aligned16(dq->codes) || !aligned16(dq->absmax2) || !aligned16(dq->offset)) return QB_EALIGN;
    if (nb >= (int64_t(1) << 31)) return QB_EINVAL;
    if (need_ws) {
        if (!dq->ws) return QB_EINVAL;
        if (!aligned16(dq->ws)) return QB_EALIGN;
        if (dq->ws_bytes < kBinBytes + round_up((size_t)nb * sizeof(float), 256)) return QB_EWORKSPACE;
    }
    return QB_OK;
}

bool finite(double v) { return std::isfinite(v); }
bool unit(double v) { return v >= 0 && v < 1; }    // [0, 1)

// Hyperparameter checks per optimizer kind (the ranges their definitions need).
// The kinds with a never-negative state (v; RMSprop's one state), which may
// hold it in QB_UDYN8.
bool has_nonneg_state(qb_optimizer k) { return k == QB_ADAMW || k == QB_ADAM || k == QB_LAMB || k == QB_RMSPROP; }

bool valid_optim(const qb_optim_hparams* hp)
{
    if (!hp || hp->step < 1 || !finite(hp->lr) || hp->lr < 0 || !finite(hp->weight_decay) || hp->weight_decay < 0)
        return false;
    if (hp->v_code != QB_DYN8 && !(hp->v_code == QB_UDYN8 && has_nonneg_state(hp->kind))) return false;
    switch (hp->kind) {
    case QB_ADAMW:
    case QB_ADAM: return unit(hp->beta1) && unit(hp->beta2) && finite(hp->eps) && hp->eps > 0;
    case QB_LION: return unit(hp->beta1) && unit(hp->beta2);
    case QB_SGD:
        // 8-bit SGD keeps a momentum state; Nesterov momentum needs zero dampening
        return hp->beta1 > 0 && hp->beta1 < 1 && hp->dampening >= 0 && hp->dampening <= 1 &&
               (hp->nesterov == 0 || (hp->nesterov == 1 && hp->dampening == 0));
    case QB_RMSPROP: return unit(hp->beta2) && finite(hp->eps) && hp->eps > 0;
    case QB_LAMB: return unit(hp->beta1) && unit(hp->beta2) && finite(hp->eps) && hp->eps > 0;
    case QB_LARS: return unit(hp->beta1) && finite(hp->trust_coefficient) && hp->trust_coefficient > 0;
    default: return false;
    }
}

qb_optim_hparams as_optim(const qb_adamw_hparams* hp)
{
    qb_optim_hparams o{};
    o.kind = QB_ADAMW;
    o.lr = hp->lr;
    o.beta1 = hp->beta1;
    o.beta2 = hp->beta2;
    o.eps = hp->eps;
    o.weight_decay = hp->weight_decay;
    o.step = hp->step;
    return o;
}

int optim_states(qb_optimizer k) { return (k == QB_ADAMW || k == QB_ADAM || k == QB_LAMB) ? 2 : 1; }
bool layerwise(qb_optimizer k) { return k == QB_LAMB || k == QB_LARS; }

// Checks one tensor of an optimizer step.  absmax1 == NULL selects binary32
// states (state1, state2 are float arrays; absmax2 must be NULL too).
qb_status check_optim_tensor(bool two, const void* p, const void* g, const void* s1, const void* s2,
                             const float* a1, const float* a2)
{
    const bool s32 = a1 == nullptr;
    if (!p || !g || !s1 || (two && !s2)) return QB_EINVAL;
    if (two && (s32 ? a2 != nullptr : a2 == nullptr)) return QB_EINVAL;
    if (p == g) return QB_EINVAL;
    if (!aligned16(p) || !aligned16(g) || !aligned16(s1) || (two && !aligned16(s2))) return QB_EALIGN;
    if (!s32 && (!aligned16(a1) || (two && !aligned16(a2)))) return QB_EALIGN;
    return QB_OK;
}

// Parameter / gradient dtype pairs of the optimizer steps: binary32
// parameters with any gradient dtype, 16-bit parameters with the same dtype.
qb_status check_optim_dtypes(qb_dtype pdt, qb_dtype gdt)
{
    if (!valid_dtype(pdt) || !valid_dtype(gdt)) return QB_EINVAL;
    return (pdt == QB_F32 || pdt == gdt) ? QB_OK : QB_EUNSUPPORTED;
}

// beta^t by t repeated binary64 multiplications.  Consecutive steps of the
// same beta reuse the previous power, so a training loop pays one multiply.
double beta_power(double beta, int32_t t, int slot)
{
    thread_local double last_beta[2] = {-1.0, -1.0};
    thread_local int32_t last_t[2] = {0, 0};
    thread_local double last_pow[2] = {1.0, 1.0};
    double p;
    int32_t k;
    if (last_beta[slot] == beta && last_t[slot] <= t) {
        p = last_pow[slot];
        k = last_t[slot];
    } else {
        p = 1.0;
        k = 0;
    }
    for (; k < t; ++k) p *= beta;
    last_beta[slot] = beta;
    last_t[slot] = t;
    last_pow[slot] = p;
    return p;
}

// Per-element scalars: computed in binary64, each rounded once to binary32.
OptScalars prepare(const qb_optim_hparams& hp)
{
    OptScalars s{};
    s.b1 = (float)hp.beta1;
    s.ob1 = (float)(1.0 - hp.beta1);
    s.b2 = (float)hp.beta2;
    s.ob2 = (float)(1.0 - hp.beta2);
    s.dec = (float)(1.0 - hp.lr * hp.weight_decay);
    s.eps = (float)hp.eps;
    s.wd = (float)hp.weight_decay;
    s.lr = (float)hp.lr;
    s.omd = (float)(1.0 - hp.dampening);
    if (hp.kind == QB_ADAMW || hp.kind == QB_ADAM || hp.kind == QB_LAMB) {
        const double p1 = beta_power(hp.beta1, hp.step, 0);
        const double p2 = beta_power(hp.beta2, hp.step, 1);
        s.s1 = (float)((hp.kind == QB_LAMB ? 1.0 : hp.lr) / (1.0 - p1));   // LAMB: the direction without lr
        s.s2 = (float)(1.0 / std::sqrt(1.0 - p2));
    }
    s.flags = (hp.nesterov ? kOptNesterov : 0) | (hp.step == 1 ? kOptFirstStep : 0);
    return s;
}

// Checks one tensor of a dequantization and fills its descriptor (tile_begin
// left 0); dq_mode: -1 = not fixed yet, 0 = plain, 1 = nested (all tensors of
// a grouped call must agree).
qb_status dequant_desc(const uint8_t* codes, const float* absmax, const uint8_t* c2, const float* absmax2,
                              const float* offset, int32_t blocksize2, int64_t n, void* y, int32_t blocksize,
                              int* dq_mode, DequantDesc* out)
{
    if (n < 0) return QB_EINVAL;
    const int64_t nb = nblocks(n, blocksize);
    if (nb >= (int64_t(1) << 31)) return QB_EINVAL;
    if (!codes || !y) return QB_EINVAL;
    if (!aligned16(codes) || !aligned16(y)) return QB_EALIGN;
    const int mode = c2 ? 1 : 0;
    if (*dq_mode >= 0 && *dq_mode != mode) return QB_EUNSUPPORTED;
    *dq_mode = mode;
    if (mode) {
        if (absmax) return QB_EINVAL;
        qb_dq tmp{const_cast<uint8_t*>(c2), const_cast<float*>(absmax2), const_cast<float*>(offset), blocksize2,
                  nullptr, 0};
        qb_status st = check_dq(&tmp, nb, false);
        if (st != QB_OK) return st;
    } else {
        if (!absmax) return QB_EINVAL;
        if (!aligned16(absmax)) return QB_EALIGN;
    }
    *out = DequantDesc{codes, absmax, c2, absmax2, offset, y, n, 0};
    return QB_OK;
}

// Appends the device tables of a multi-tensor launch (descriptors, the first
// tile of every tensor, the coarse bucket index: see TileMap) to the host
// staging buffer at byte `at` (a multiple of 16), for a copy to ws + at; fills
// *map with those device addresses.  `tiles` is the total.
template <class Desc>
void stage_tile_map(std::vector<unsigned char>& staging, size_t at, const std::vector<Desc>& table, int64_t tiles,
                    int32_t count, void* ws, TileMap<Desc>* map)
{
    thread_local std::vector<int64_t> begins;
    thread_local std::vector<int32_t> buckets;
    begins.clear();
    buckets.clear();
    for (const Desc& d : table) begins.push_back(d.tile_begin);
    begins.push_back(tiles);
    // the smallest bucket width 2^shift that needs at most
    // max_tile_buckets(count) buckets; bucket k starts at tile k << shift
    const int32_t used = (int32_t)table.size();
    int shift = 0;
    while (((tiles - 1) >> shift) + 1 > max_tile_buckets(count)) ++shift;
    const int64_t nbk = ((tiles - 1) >> shift) + 1;
    for (int64_t k = 0, i = 0; k < nbk; ++k) {
        const int64_t first = k << shift;
        while (begins[i + 1] <= first) ++i;          // begins[used] = tiles > first
        buckets.push_back((int32_t)i);
    }
    buckets.push_back(used - 1);
    const size_t dbytes = table.size() * sizeof(Desc), bbytes = begins.size() * sizeof(int64_t),
                 kbytes = buckets.size() * sizeof(int32_t);
    staging.resize(at + dbytes + bbytes + kbytes);
    std::memcpy(staging.data() + at, table.data(), dbytes);
    std::memcpy(staging.data() + at + dbytes, begins.data(), bbytes);
    std::memcpy(staging.data() + at + dbytes + bbytes, buckets.data(), kbytes);
    unsigned char* w = static_cast<unsigned char*>(ws) + at;
    *map = TileMap<Desc>{reinterpret_cast<const Desc*>(w), reinterpret_cast<const int64_t*>(w + dbytes),
                         reinterpret_cast<const int32_t*>(w + dbytes + bbytes), used, shift};
}

// One copy of the staged tables to ws on stream s (from pageable memory: the
// copy has read the host buffer when hipMemcpyAsync returns).
qb_status copy_staging(const std::vector<unsigned char>& staging, void* ws, hipStream_t s)
{
    return hipMemcpyAsync(ws, staging.data(), staging.size(), hipMemcpyHostToDevice, s) == hipSuccess ? QB_OK
                                                                                                       : QB_EHIP;
}

// Bytes of one multi-tensor table region (qb_multi_tensor_workspace_bytes).
size_t map_region_bytes(int32_t count)
{
    return count > 0 ? round_up((size_t)count * 64 + ((size_t)count + 1) * sizeof(int64_t) +
                                    ((size_t)max_tile_buckets(count) + 1) * sizeof(int32_t), 256)
                     : 0;
}

// Norm groups of a tensor: kNormGroupTiles optimizer tiles each.
int64_t norm_groups(int64_t n, int32_t B)
{
    return (adamw_tiles(n, B) + kNormGroupTiles - 1) / kNormGroupTiles;
}

// Workspace of a layer-wise step: the tile map region, the group map region,
// then 16 bytes of partial sums per group, then one float S per tensor.
// Returns the bytes; with ws given, sets *part and *trust to their addresses.
size_t layerwise_ws_layout(int32_t count, int64_t groups, void* ws, double** part, float** trust)
{
    const size_t m = 2 * map_region_bytes(count);
    const size_t pb = round_up((size_t)groups * 2 * sizeof(double), 256);
    if (ws) {
        *part = reinterpret_cast<double*>(static_cast<char*>(ws) + m);
        *trust = reinterpret_cast<float*>(static_cast<char*>(ws) + m + pb);
    }
    return m + pb + round_up((size_t)count * sizeof(float), 256);
}

int64_t quant_tiles(int64_t n, int32_t B, int bits)
{
    const int64_t t = quant_tile_elems(B, bits);
    return (n + t - 1) / t;
}

// Checks one tensor of a quantization; nested: -1 = not fixed yet, 0 =
// plain, 1 = nested (all tensors of a grouped call must agree).
qb_status check_quant_tensor(const void* x, uint8_t* codes, float* absmax, uint8_t* c2, float* absmax2,
                             float* offset, int64_t n, int32_t blocksize, int32_t blocksize2, int* nested)
{
    if (n < 0) return QB_EINVAL;
    const int64_t nb = nblocks(n, blocksize);
    if (nb >= (int64_t(1) << 31)) return QB_EINVAL;
    if (!x || !codes) return QB_EINVAL;
    if (!aligned16(x) || !aligned16(codes)) return QB_EALIGN;
    const int mode = c2 ? 1 : 0;
    if (*nested >= 0 && *nested != mode) return QB_EUNSUPPORTED;
    *nested = mode;
    if (mode) {
        if (absmax) return QB_EINVAL;
        qb_dq tmp{c2, absmax2, offset, blocksize2, nullptr, 0};
        return check_dq(&tmp, nb, false);
    }
    if (!absmax) return QB_EINVAL;
    return aligned16(absmax) ? QB_OK : QB_EALIGN;
}

int64_t dequant_tiles(int64_t n, int64_t tile) { return (n + tile - 1) / tile; }

// Per-device resources of the paged step: the two copy streams (default
// priority) and the events that order the staging slots; created on first
// use and kept until the process ends.
struct PagedRes {
    hipStream_t h2d = nullptr, d2h = nullptr;
    hipEvent_t start = nullptr, done = nullptr;
    hipEvent_t in[2] = {nullptr, nullptr}, kern[2] = {nullptr, nullptr}, out[2] = {nullptr, nullptr};
};

PagedRes* paged_resources()
{
    static std::mutex mu;
    static std::vector<PagedRes*> per_dev;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1, nullptr);
    if (per_dev[dev]) return per_dev[dev];
    PagedRes* r = new PagedRes;
    bool ok = hipStreamCreateWithFlags(&r->h2d, hipStreamNonBlocking) == hipSuccess &&
              hipStreamCreateWithFlags(&r->d2h, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&r->start, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&r->done, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; ok && i < 2; ++i)
        ok = hipEventCreateWithFlags(&r->in[i], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&r->kern[i], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&r->out[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) return nullptr;                       // (kept: a later call retries nothing, reports QB_EHIP)
    per_dev[dev] = r;
    return r;
}

// True if p points into pinned (page-locked) host memory.
bool pinned_host(const void* p)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();                   // pageable memory: clear the error the query left
        return false;
    }
    return a.type == hipMemoryTypeHost;
}

// Bytes of one staging region of the paged step.
size_t paged_region(int64_t P, int32_t B, bool codes)
{
    return codes ? round_up((size_t)P, 256) : round_up((size_t)((P + B - 1) / B) * sizeof(float), 256);
}

}  // namespace

extern "C" {

const char* qb_status_string(qb_status s)
{
    switch (s) {
    case QB_OK: return "ok";
    case QB_EINVAL: return "invalid argument";
    case QB_EALIGN: return "device pointer not 16-byte aligned";
    case QB_EUNSUPPORTED: return "unsupported combination";
    case QB_EHIP: return "HIP runtime error";
    case QB_EWORKSPACE: return "workspace too small";
    case QB_EINIT: return "constant tables could not be built or uploaded";
    default: return "unknown status";
    }
}

size_t qb_dq_workspace_bytes(int64_t n, int32_t blocksize)
{
    if (n < 0 || !pow2_block(blocksize)) return 0;
    return kBinBytes + round_up((size_t)nblocks(n, blocksize) * sizeof(float), 256);
}

size_t qb_multi_tensor_workspace_bytes(int32_t count)
{
    // descriptors, count + 1 int64 first-tile numbers, then the coarse bucket
    // index (max_tile_buckets(count) + 1 int32 entries)
    if (count <= 0) return 0;
    return (size_t)count * sizeof(TensorDesc) + ((size_t)count + 1) * sizeof(int64_t) +
           ((size_t)max_tile_buckets(count) + 1) * sizeof(int32_t);
}

int32_t qb_codebook(qb_code code, float* out)
{
    const QbTables* t = host_tables();
    if (!t || !out || !(valid_code(code) || code == QB_UDYN8)) return -1;
    if (code == QB_DYN8 || code == QB_UDYN8) {
        std::memcpy(out, code == QB_DYN8 ? t->dyn8 : t->udyn8, sizeof(t->dyn8));
        return 256;
    }
    std::memcpy(out, code == QB_NF4 ? t->nf4 : t->fp4, 16 * sizeof(float));
    return 16;
}

int32_t qb_encoder_table(qb_code code, uint32_t* out, int32_t capacity)
{
    const QbTables* t = host_tables();
    if (!t || !(valid_code(code) || code == QB_UDYN8) || capacity < 0 || (capacity > 0 && !out)) return -1;
    if (code == QB_UDYN8) {
        for (int32_t i = 0; i < kUDynLutN && i < capacity; ++i) {
            const int c = t->udyn8_base[i];
            out[2 * i] = t->udyn8_thr[c];
            out[2 * i + 1] = (uint32_t)c;
        }
        return kUDynLutN;
    }
    if (code == QB_DYN8) {
        for (int32_t i = 0; i < 2 * kDynLutN && i < capacity; ++i) {
            const int c = t->dyn8_base[i / kDynLutN][i % kDynLutN];
            out[2 * i] = t->dyn8_thr[c];
            out[2 * i + 1] = (uint32_t)c;
        }
        return 2 * kDynLutN;
    }
    const LutEntry* src = code == QB_NF4 ? t->nf4_lut : t->fp4_lut;
    for (int32_t i = 0; i < k4LutN && i < capacity; ++i) {
        out[2 * i] = src[i].t;
        out[2 * i + 1] = src[i].payload;
    }
    return k4LutN;
}

qb_status qb_quantize(const void* x, qb_dtype xdt, int64_t n, qb_code code, int32_t blocksize,
                      uint8_t* codes, float* absmax, const qb_dq* dq, void* stream)
{
    if (n < 0 || !valid_dtype(xdt) || !valid_code(code) || !pow2_block(blocksize)) return QB_EINVAL;
    if (n == 0) return QB_OK;
    int nested = dq ? 1 : 0;
    if (dq && !dq->codes) return QB_EINVAL;
    qb_status st = check_quant_tensor(x, codes, absmax, dq ? dq->codes : nullptr, dq ? dq->absmax2 : nullptr,
                                      dq ? dq->offset : nullptr, n, blocksize, dq ? dq->blocksize2 : 0, &nested);
    if (st != QB_OK) return st;
    const int64_t nb = nblocks(n, blocksize);
    if (dq) {
        st = check_dq(dq, nb, true);
        if (st != QB_OK) return st;
    }
    if (!device_tables()) return QB_EINIT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int bits = is4(code) ? 4 : 8, c4 = is4(code) ? code4_index(code) : 0;
    if (!dq)
        return hip_status(launch_quant(QuantDesc{x, codes, absmax, nullptr, n, 0, {0, 0}}, nullptr,
                                       quant_tiles(n, blocksize, bits), bits, c4, blocksize, (int)xdt, false, nullptr, s));
    // nested: bins, then the fp32 absmax, in the workspace
    unsigned long long* bins = static_cast<unsigned long long*>(dq->ws);
    float* first = reinterpret_cast<float*>(static_cast<char*>(dq->ws) + kBinBytes);
    const QuantDesc d1{x, codes, first, nullptr, n, 0, {0, 0}};
    const QuantDesc d2{first, dq->codes, dq->absmax2, dq->offset, nb, 0, {0, 0}};
    hipError_t e = launch_clear_bins(bins, 1, s);
    if (e == hipSuccess)
        e = launch_quant(d1, nullptr, quant_tiles(n, blocksize, bits), bits, c4, blocksize, (int)xdt, false, bins, s);
    if (e == hipSuccess) e = launch_dq_mean(d2, nullptr, 1, bins, s);
    if (e == hipSuccess)
        e = launch_quant(d2, nullptr, quant_tiles(nb, dq->blocksize2, 8), 8, 0, dq->blocksize2, QB_F32, true, nullptr, s);
    return hip_status(e);
}

qb_status qb_normalize(const void* x, qb_dtype xdt, int64_t n, const float* absmax, int32_t blocksize, float* out,
                       void* stream)
{
    if (n < 0 || !valid_dtype(xdt) || blocksize < 1) return QB_EINVAL;
    if (n == 0) return QB_OK;
    if (!x || !absmax || !out) return QB_EINVAL;
    if (!aligned16(x) || !aligned16(absmax) || !aligned16(out)) return QB_EALIGN;
    if ((n + 255) / 256 >= (int64_t(1) << 31)) return QB_EINVAL;
    return hip_status(launch_normalize(x, (int)xdt, n, absmax, blocksize, out, static_cast<hipStream_t>(stream)));
}

size_t qb_multi_tensor_quantize_workspace_bytes(const qb_quant_tensor* tensors, int32_t count, int32_t blocksize)
{
    if (count <= 0 || !tensors || !pow2_block(blocksize)) return 0;
    bool nested = false;
    size_t temps = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (tensors[i].n < 0) return 0;
        if (tensors[i].c2) nested = true;
        temps += round_up((size_t)nblocks(tensors[i].n, blocksize) * sizeof(float), 256);
    }
    const size_t m = map_region_bytes(count);
    return nested ? 2 * m + (size_t)count * kBinBytes + temps : m;
}

qb_status qb_multi_tensor_quantize(const qb_quant_tensor* tensors, int32_t count, qb_dtype xdt, qb_code code,
                                   int32_t blocksize, int32_t blocksize2, void* ws, size_t ws_bytes, void* stream)
{
    if (count < 0 || !valid_dtype(xdt) || !valid_code(code) || !pow2_block(blocksize)) return QB_EINVAL;
    if (count == 0) return QB_OK;
    if (!tensors || !ws) return QB_EINVAL;
    if (!aligned16(ws)) return QB_EALIGN;
    thread_local std::vector<QuantDesc> t1, t2;
    t1.clear();
    t2.clear();
    int nested = -1;
    int64_t tiles1 = 0, tiles2 = 0;
    for (int32_t i = 0; i < count; ++i) {
        const qb_quant_tensor& t = tensors[i];
        qb_status st = check_quant_tensor(t.x, t.codes, t.absmax, t.c2, t.absmax2, t.offset, t.n, blocksize,
                                          blocksize2, &nested);
        if (st != QB_OK) return st;
    }
    if (ws_bytes < qb_multi_tensor_quantize_workspace_bytes(tensors, count, blocksize)) return QB_EWORKSPACE;
    const size_t m = map_region_bytes(count);
    unsigned char* const w = static_cast<unsigned char*>(ws);
    unsigned long long* const bins = reinterpret_cast<unsigned long long*>(w + 2 * m);
    unsigned char* temp = w + 2 * m + (size_t)count * kBinBytes;
    for (int32_t i = 0; i < count; ++i) {
        const qb_quant_tensor& t = tensors[i];
        if (t.n == 0) continue;
        const int64_t nb = nblocks(t.n, blocksize);
        if (nested == 1) {
            float* first = reinterpret_cast<float*>(temp);
            temp += round_up((size_t)nb * sizeof(float), 256);
            t1.push_back(QuantDesc{t.x, t.codes, first, nullptr, t.n, tiles1, {0, 0}});
            t2.push_back(QuantDesc{first, t.c2, t.absmax2, t.offset, nb, tiles2, {0, 0}});
            tiles2 += quant_tiles(nb, blocksize2, 8);
        } else {
            t1.push_back(QuantDesc{t.x, t.codes, t.absmax, nullptr, t.n, tiles1, {0, 0}});
        }
        tiles1 += quant_tiles(t.n, blocksize, is4(code) ? 4 : 8);
    }
    if (t1.empty()) return QB_OK;
    if (tiles1 >= (int64_t(1) << 31)) return QB_EINVAL;
    if (!device_tables()) return QB_EINIT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    thread_local std::vector<unsigned char> staging;
    staging.clear();
    TileMap<QuantDesc> map1, map2;
    stage_tile_map(staging, 0, t1, tiles1, count, ws, &map1);
    if (nested == 1) stage_tile_map(staging, m, t2, tiles2, count, ws, &map2);
    qb_status st = copy_staging(staging, ws, s);
    if (st != QB_OK) return st;
    const int bits = is4(code) ? 4 : 8, c4 = is4(code) ? code4_index(code) : 0;
    if (nested != 1)
        return hip_status(launch_quant(t1[0], &map1, tiles1, bits, c4, blocksize, (int)xdt, false, nullptr, s));
    hipError_t e = launch_clear_bins(bins, (int)t1.size(), s);
    if (e == hipSuccess) e = launch_quant(t1[0], &map1, tiles1, bits, c4, blocksize, (int)xdt, false, bins, s);
    if (e == hipSuccess) e = launch_dq_mean(t2[0], &map2, (int)t2.size(), bins, s);
    if (e == hipSuccess) e = launch_quant(t2[0], &map2, tiles2, 8, 0, blocksize2, QB_F32, true, nullptr, s);
    return hip_status(e);
}

qb_status qb_dequantize(const uint8_t* codes, const float* absmax, const qb_dq* dq, qb_code code,
                        int32_t blocksize, int64_t n, void* y, qb_dtype ydt, void* stream)
{
    if (n < 0 || !valid_dtype(ydt) || !valid_code(code) || !pow2_block(blocksize)) return QB_EINVAL;
    if (n == 0) return QB_OK;
    int mode = dq ? 1 : 0;
    if (dq && !dq->codes) return QB_EINVAL;
    DequantDesc d;
    qb_status st = dequant_desc(codes, absmax, dq ? dq->codes : nullptr, dq ? dq->absmax2 : nullptr,
                                dq ? dq->offset : nullptr, dq ? dq->blocksize2 : 0, n, y, blocksize, &mode, &d);
    if (st != QB_OK) return st;
    if (!device_tables()) return QB_EINIT;
    const int bits = is4(code) ? 4 : 8;
    return hip_status(launch_dequant(d, nullptr, dequant_tiles(n, dequant_tile_elems(bits, false, (int)ydt)), bits,
                                     is4(code) ? code4_index(code) : 0, blocksize, dq ? dq->blocksize2 : 256,
                                     dq != nullptr, (int)ydt, static_cast<hipStream_t>(stream)));
}

qb_status qb_dequant_matmul(const void* x, qb_dtype xdt, int64_t M, int64_t K, const uint8_t* codes,
                            const float* absmax, const qb_dq* dq, qb_code code, int32_t blocksize, int64_t N,
                            void* y, void* stream)
{
    // K < 2^24: the kernel keeps a lane's offsets within a 64-row tile of x in 32 bits
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || K >= (int64_t(1) << 24) || !valid_dtype(xdt) || !is4(code) ||
        !pow2_block(blocksize))
        return QB_EINVAL;
    if (M == 0 || N == 0) return QB_OK;
    if (!x || !codes || !y) return QB_EINVAL;
    if (N > INT64_MAX / K) return QB_EINVAL;
    const int64_t nb = nblocks(N * K, blocksize);
    if (dq) {
        if (absmax) return QB_EINVAL;
        qb_status st = check_dq(dq, nb, false);
        if (st != QB_OK) return st;
    } else if (!absmax) {
        return QB_EINVAL;
    }
    if (!aligned16(x) || !aligned16(codes) || !aligned16(y) || (absmax && !aligned16(absmax))) return QB_EALIGN;
    if (!device_tables()) return QB_EINIT;
    return hip_status(launch_dq4_matmul(x, (int)xdt, M, K, codes, absmax, dq ? dq->codes : nullptr,
                                        dq ? dq->absmax2 : nullptr, dq ? dq->offset : nullptr, blocksize,
                                        dq ? dq->blocksize2 : 256, code4_index(code), N, y,
                                        static_cast<hipStream_t>(stream)));
}

qb_status qb_dequant_matmul_grouped(const void* x, qb_dtype xdt, int64_t M, int64_t K, const qb_matmul_weight* weights,
                                    int32_t count, qb_code code, int32_t blocksize, int32_t blocksize2, void* stream)
{
    if (count < 0 || count > QB_MATMUL_GROUP_MAX || M < 0 || K <= 0 || K % 32 != 0 || K >= (int64_t(1) << 24) ||
        !valid_dtype(xdt) || !is4(code) || !pow2_block(blocksize))
        return QB_EINVAL;
    if (count == 0 || M == 0) return QB_OK;
    if (!weights || !x) return QB_EINVAL;
    if (!aligned16(x)) return QB_EALIGN;
    MmWeight w[kMmGroupMax];
    int n = 0, mode = -1;
    for (int32_t i = 0; i < count; ++i) {
        const qb_matmul_weight& t = weights[i];
        if (t.N < 0 || t.N > INT64_MAX / K) return QB_EINVAL;
        if (t.N == 0) continue;                        // skipped, whatever its pointers
        DequantDesc d;
        qb_status st = dequant_desc(t.codes, t.absmax, t.c2, t.absmax2, t.offset, blocksize2, t.N * K, t.y, blocksize,
                                    &mode, &d);
        if (st != QB_OK) return st;
        w[n++] = MmWeight{t.codes, t.absmax, t.c2, t.absmax2, t.offset, t.y, t.N};
    }
    if (n == 0) return QB_OK;
    if (!device_tables()) return QB_EINIT;
    return hip_status(launch_dq4_matmul_grouped(x, (int)xdt, M, K, w, n, blocksize, mode == 1 ? blocksize2 : 256,
                                                code4_index(code), static_cast<hipStream_t>(stream)));
}

qb_status qb_multi_tensor_dequantize(const qb_dequant_tensor* tensors, int32_t count, qb_code code,
                                     int32_t blocksize, int32_t blocksize2, qb_dtype ydt, void* ws, size_t ws_bytes,
                                     void* stream)
{
    if (count < 0 || !valid_dtype(ydt) || !valid_code(code) || !pow2_block(blocksize)) return QB_EINVAL;
    if (count == 0) return QB_OK;
    if (!tensors || !ws) return QB_EINVAL;
    if (!aligned16(ws)) return QB_EALIGN;
    if (ws_bytes < qb_multi_tensor_workspace_bytes(count)) return QB_EWORKSPACE;
    thread_local std::vector<DequantDesc> table;
    table.clear();
    int mode = -1;
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) {
        const qb_dequant_tensor& t = tensors[i];
        DequantDesc d;
        qb_status st = dequant_desc(t.codes, t.absmax, t.c2, t.absmax2, t.offset, blocksize2, t.n, t.y, blocksize,
                                    &mode, &d);
        if (st != QB_OK) return st;
        if (t.n == 0) continue;
        d.tile_begin = tiles;
        table.push_back(d);
        tiles += dequant_tiles(t.n, dequant_tile_elems(is4(code) ? 4 : 8, true, (int)ydt));
    }
    if (table.empty()) return QB_OK;
    if (tiles >= (int64_t(1) << 31)) return QB_EINVAL;
    if (!device_tables()) return QB_EINIT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    thread_local std::vector<unsigned char> staging;
    staging.clear();
    TileMap<DequantDesc> map;
    stage_tile_map(staging, 0, table, tiles, count, ws, &map);
    qb_status st = copy_staging(staging, ws, s);
    if (st != QB_OK) return st;
    return hip_status(launch_dequant(table[0], &map, tiles, is4(code) ? 4 : 8, is4(code) ? code4_index(code) : 0,
                                     blocksize, mode == 1 ? blocksize2 : 256, mode == 1, (int)ydt, s));
}

size_t qb_code_table_bytes(void) { return sizeof(UserCode); }

int32_t qb_linear_code(float* out)
{
    if (!out) return -1;
    linear_code(out);
    return 256;
}

qb_status qb_prepare_code(const float* values, void* table, void* stream)
{
    if (!values || !table) return QB_EINVAL;
    if (!aligned16(table)) return QB_EALIGN;
    thread_local UserCode staged;
    std::memcpy(staged.values, values, sizeof(staged.values));
    if (user_code_thresholds(staged.values, staged.thr) != 0) return QB_EINVAL;
    user_code_first(staged.thr, staged.first);
    // from pageable memory: the copy has read `staged` when hipMemcpyAsync returns
    return hipMemcpyAsync(table, &staged, sizeof(staged), hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? QB_OK
               : QB_EHIP;
}

qb_status qb_quantize_code(const void* x, qb_dtype xdt, int64_t n, const void* table, int32_t blocksize,
                           uint8_t* codes, float* absmax, void* stream)
{
    if (n < 0 || !valid_dtype(xdt) || !pow2_block(blocksize)) return QB_EINVAL;
    if (n == 0) return QB_OK;
    if (!table) return QB_EINVAL;
    if (!aligned16(table)) return QB_EALIGN;
    int nested = 0;
    qb_status st = check_quant_tensor(x, codes, absmax, nullptr, nullptr, nullptr, n, blocksize, 0, &nested);
    if (st != QB_OK) return st;
    return hip_status(launch_quant_user(QuantDesc{x, codes, absmax, nullptr, n, 0, {0, 0}}, quant_tiles(n, blocksize, 8),
                                        blocksize, (int)xdt, static_cast<const UserCode*>(table),
                                        static_cast<hipStream_t>(stream)));
}

qb_status qb_dequantize_code(const uint8_t* codes, const float* absmax, const void* table, int32_t blocksize,
                             int64_t n, void* y, qb_dtype ydt, void* stream)
{
    if (n < 0 || !valid_dtype(ydt) || !pow2_block(blocksize)) return QB_EINVAL;
    if (n == 0) return QB_OK;
    if (!table) return QB_EINVAL;
    if (!aligned16(table)) return QB_EALIGN;
    int mode = 0;
    DequantDesc d;
    qb_status st = dequant_desc(codes, absmax, nullptr, nullptr, nullptr, 0, n, y, blocksize, &mode, &d);
    if (st != QB_OK) return st;
    return hip_status(launch_dequant_user(d, dequant_tiles(n, dequant_tile_elems(8, false, (int)ydt)), blocksize, (int)ydt,
                                          static_cast<const UserCode*>(table), static_cast<hipStream_t>(stream)));
}

size_t qb_quantile_workspace_bytes(int64_t n)
{
    // the chunks' order statistics (float [257][nchunks]), then their means
    // (double [257])
    if (n <= 0) return 0;
    const int64_t nchunks = (n + kQuantileChunk - 1) / kQuantileChunk;
    return round_up((size_t)nchunks * 257 * sizeof(float), 256) + 257 * sizeof(double);
}

qb_status qb_estimate_quantiles(const void* x, qb_dtype xdt, int64_t n, void* table, double* averages, void* ws,
                                size_t ws_bytes, void* stream)
{
    if (n < 1 || !valid_dtype(xdt)) return QB_EINVAL;
    if (!x || !table || !ws) return QB_EINVAL;
    if (!aligned16(x) || !aligned16(table) || !aligned16(ws) || (averages && !aligned16(averages))) return QB_EALIGN;
    if ((n + kQuantileChunk - 1) / kQuantileChunk >= (int64_t(1) << 31)) return QB_EINVAL;
    if (ws_bytes < qb_quantile_workspace_bytes(n)) return QB_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nchunks = (n + kQuantileChunk - 1) / kQuantileChunk;
    float* E = static_cast<float*>(ws);
    double* A = reinterpret_cast<double*>(static_cast<char*>(ws) + round_up((size_t)nchunks * 257 * sizeof(float), 256));
    hipError_t e = launch_chunk_quantiles(x, (int)xdt, n, E, s);
    if (e == hipSuccess) e = launch_quantile_code(E, nchunks, A, averages, static_cast<UserCode*>(table), s);
    return hip_status(e);
}

qb_status qb_optimizer8bit_step(const qb_optim_hparams* hp, void* p, qb_dtype pdt, const void* g, qb_dtype gdt,
                                int64_t n, uint8_t* state1, uint8_t* state2, float* absmax1, float* absmax2,
                                int32_t blocksize, void* stream)
{
    if (n < 0 || !valid_dtype(pdt) || !valid_dtype(gdt) || !pow2_block(blocksize) || !valid_optim(hp))
        return QB_EINVAL;
    if (check_optim_dtypes(pdt, gdt) != QB_OK || layerwise(hp->kind)) return QB_EUNSUPPORTED;
    if (n == 0) return QB_OK;
    const bool two = optim_states(hp->kind) == 2;
    if (!two) {
        state2 = nullptr;
        absmax2 = nullptr;
    }
    if (nblocks(n, blocksize) >= (int64_t(1) << 31)) return QB_EINVAL;
    qb_status st = check_optim_tensor(two, p, g, state1, state2, absmax1, absmax2);
    if (st != QB_OK) return st;
    if (!device_tables()) return QB_EINIT;
    TensorDesc d{p, g, state1, state2, absmax1, absmax2, n, 0};
    return hip_status(launch_optim8((int)hp->kind, d, nullptr, adamw_tiles(n, blocksize), blocksize, (int)pdt,
                                    (int)gdt, prepare(*hp), nullptr, hp->v_code == QB_UDYN8,
                                    static_cast<hipStream_t>(stream)));
}

size_t qb_optimizer_workspace_bytes(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count,
                                    int32_t blocksize)
{
    if (!hp || count < 0 || (count > 0 && !tensors) || !pow2_block(blocksize)) return 0;
    if (!layerwise(hp->kind)) return qb_multi_tensor_workspace_bytes(count);
    int64_t groups = 0;
    for (int32_t i = 0; i < count; ++i) {
        if (tensors[i].n < 0) return 0;
        groups += norm_groups(tensors[i].n, blocksize);
    }
    return layerwise_ws_layout(count, groups, nullptr, nullptr, nullptr);
}

qb_status qb_multi_tensor_optimizer_step(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count,
                                         qb_dtype pdt, qb_dtype gdt, int32_t blocksize, void* ws, size_t ws_bytes,
                                         void* stream)
{
    if (count < 0 || !valid_dtype(pdt) || !valid_dtype(gdt) || !pow2_block(blocksize) || !valid_optim(hp))
        return QB_EINVAL;
    if (check_optim_dtypes(pdt, gdt) != QB_OK) return QB_EUNSUPPORTED;
    if (count == 0) return QB_OK;
    if (!tensors || !ws) return QB_EINVAL;
    if (!aligned16(ws)) return QB_EALIGN;
    if (ws_bytes < qb_multi_tensor_workspace_bytes(count)) return QB_EWORKSPACE;
    const bool two = optim_states(hp->kind) == 2;
    thread_local std::vector<TensorDesc> table;
    table.clear();
    int64_t tiles = 0;
    for (int32_t i = 0; i < count; ++i) {
        const qb_tensor& t = tensors[i];
        if (t.n < 0) return QB_EINVAL;
        if (t.n == 0) continue;
        if (nblocks(t.n, blocksize) >= (int64_t(1) << 31)) return QB_EINVAL;
        qb_status st = check_optim_tensor(two, t.p, t.g, t.m, t.v, t.absmax_m, t.absmax_v);
        if (st != QB_OK) return st;
        table.push_back(TensorDesc{t.p, t.g, t.m, two ? t.v : nullptr, t.absmax_m, two ? t.absmax_v : nullptr, t.n,
                                   tiles});
        tiles += adamw_tiles(t.n, blocksize);
    }
    if (table.empty()) return QB_OK;
    if (tiles >= (int64_t(1) << 31)) return QB_EINVAL;
    double* part = nullptr;
    float* trust = nullptr;
    thread_local std::vector<TensorDesc> gtable;      // the same tensors, numbered by norm group
    int64_t groups = 0;
    if (layerwise(hp->kind)) {
        gtable = table;
        for (TensorDesc& d : gtable) {
            d.tile_begin = groups;
            groups += norm_groups(d.n, blocksize);
        }
        if (ws_bytes < layerwise_ws_layout(count, groups, ws, &part, &trust)) return QB_EWORKSPACE;
    }
    if (!device_tables()) return QB_EINIT;
    hipStream_t s = static_cast<hipStream_t>(stream);
    thread_local std::vector<unsigned char> staging;
    staging.clear();
    TileMap<TensorDesc> map;
    const OptScalars hs = prepare(*hp);
    if (layerwise(hp->kind)) {
        TileMap<TensorDesc> gmap;
        stage_tile_map(staging, 0, table, tiles, count, ws, &map);
        stage_tile_map(staging, map_region_bytes(count), gtable, groups, count, ws, &gmap);
        qb_status st = copy_staging(staging, ws, s);
        if (st != QB_OK) return st;
        const bool uv = hp->v_code == QB_UDYN8;
        hipError_t e = launch_trust_norms((int)hp->kind, gmap, groups, blocksize, (int)pdt, (int)gdt, hs, part, uv, s);
        if (e == hipSuccess)
            e = launch_trust_scalars((int)hp->kind, gmap, part, hp->lr, hp->weight_decay, hp->trust_coefficient,
                                     trust, s);
        if (e == hipSuccess)
            e = launch_optim8((int)hp->kind, table[0], &map, tiles, blocksize, (int)pdt, (int)gdt, hs, trust, uv, s);
        return hip_status(e);
    }
    stage_tile_map(staging, 0, table, tiles, count, ws, &map);
    qb_status st = copy_staging(staging, ws, s);
    if (st != QB_OK) return st;
    return hip_status(
        launch_optim8((int)hp->kind, table[0], &map, tiles, blocksize, (int)pdt, (int)gdt, hs, nullptr,
                      hp->v_code == QB_UDYN8, s));
}

qb_status qb_adamw8bit_step(float* p, const void* g, qb_dtype gdt, int64_t n, uint8_t* m, uint8_t* v,
                            float* absmax_m, float* absmax_v, int32_t blocksize, const qb_adamw_hparams* hp,
                            void* stream)
{
    if (!hp) return QB_EINVAL;
    const qb_optim_hparams o = as_optim(hp);
    return qb_optimizer8bit_step(&o, p, QB_F32, g, gdt, n, m, v, absmax_m, absmax_v, blocksize, stream);
}

qb_status qb_multi_tensor_step(const qb_tensor* tensors, int32_t count, qb_dtype gdt, int32_t blocksize,
                               const qb_adamw_hparams* hp, void* ws, size_t ws_bytes, void* stream)
{
    if (!hp) return QB_EINVAL;
    const qb_optim_hparams o = as_optim(hp);
    return qb_multi_tensor_optimizer_step(&o, tensors, count, QB_F32, gdt, blocksize, ws, ws_bytes, stream);
}

qb_status qb_multi_tensor_step_noalloc(const qb_tensor* tensors, int32_t count, qb_dtype gdt, int32_t blocksize,
                                       const qb_adamw_hparams* hp, void* stream)
{
    if (!hp || count < 0) return QB_EINVAL;
    if (count > kScratchMaxTensors || qb_multi_tensor_workspace_bytes(count) > kScratchBytes) return QB_EWORKSPACE;
    if (count == 0) return QB_OK;
    void* ws = device_scratch();
    if (!ws) return QB_EHIP;
    return qb_multi_tensor_step(tensors, count, gdt, blocksize, hp, ws, kScratchBytes, stream);
}

size_t qb_paged_workspace_bytes(int64_t page_params, int32_t blocksize)
{
    if (!pow2_block(blocksize) || page_params <= 0 || page_params % blocksize != 0) return 0;
    return 2 * (2 * paged_region(page_params, blocksize, true) + 2 * paged_region(page_params, blocksize, false));
}

qb_status qb_paged_optimizer_step(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count, qb_dtype pdt,
                                  qb_dtype gdt, int32_t blocksize, int64_t page_params, void* ws, size_t ws_bytes,
                                  void* stream)
{
    if (count < 0 || !valid_dtype(pdt) || !valid_dtype(gdt) || !pow2_block(blocksize) || !valid_optim(hp))
        return QB_EINVAL;
    if (check_optim_dtypes(pdt, gdt) != QB_OK || layerwise(hp->kind)) return QB_EUNSUPPORTED;
    if (page_params <= 0 || page_params % blocksize != 0 || page_params >= (int64_t(1) << 31)) return QB_EINVAL;
    if (count == 0) return QB_OK;
    if (!tensors || !ws) return QB_EINVAL;
    if (!aligned16(ws)) return QB_EALIGN;
    if (ws_bytes < qb_paged_workspace_bytes(page_params, blocksize)) return QB_EWORKSPACE;
    const bool two = optim_states(hp->kind) == 2;
    for (int32_t i = 0; i < count; ++i) {
        const qb_tensor& t = tensors[i];
        if (t.n < 0) return QB_EINVAL;
        if (t.n == 0) continue;
        if (nblocks(t.n, blocksize) >= (int64_t(1) << 31)) return QB_EINVAL;
        if (!t.absmax_m || (two && !t.absmax_v)) return QB_EUNSUPPORTED;      // 8-bit states only
        qb_status st = check_optim_tensor(two, t.p, t.g, t.m, two ? t.v : nullptr, t.absmax_m,
                                          two ? t.absmax_v : nullptr);
        if (st != QB_OK) return st;
        if (!pinned_host(t.m) || !pinned_host(t.absmax_m) ||
            (two && (!pinned_host(t.v) || !pinned_host(t.absmax_v))))
            return QB_EINVAL;
    }
    if (!device_tables()) return QB_EINIT;
    PagedRes* r = paged_resources();
    if (!r) return QB_EHIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const OptScalars hs = prepare(*hp);
    const int64_t P = page_params;
    const size_t cb = paged_region(P, blocksize, true), ab = paged_region(P, blocksize, false);
    const size_t slot_bytes = 2 * cb + 2 * ab;
    auto ck = [](hipError_t e) { return e == hipSuccess; };
    // the copies start after the work already on `stream`
    if (!ck(hipEventRecord(r->start, s)) || !ck(hipStreamWaitEvent(r->h2d, r->start, 0)) ||
        !ck(hipStreamWaitEvent(r->d2h, r->start, 0)))
        return QB_EHIP;
    int64_t page = 0;
    for (int32_t i = 0; i < count; ++i) {
        const qb_tensor& t = tensors[i];
        for (int64_t off = 0; off < t.n; off += P, ++page) {
            const int slot = (int)(page & 1);
            const int64_t n = t.n - off < P ? t.n - off : P;
            const int64_t b0 = off / blocksize, nb = (n + blocksize - 1) / blocksize;
            char* base = static_cast<char*>(ws) + slot * slot_bytes;
            uint8_t* m = reinterpret_cast<uint8_t*>(base);
            uint8_t* v = reinterpret_cast<uint8_t*>(base + cb);
            float* am = reinterpret_cast<float*>(base + 2 * cb);
            float* av = reinterpret_cast<float*>(base + 2 * cb + ab);
            // host to device, once the slot's previous page has been copied back
            bool ok = page < 2 || ck(hipStreamWaitEvent(r->h2d, r->out[slot], 0));
            ok = ok && ck(hipMemcpyAsync(m, t.m + off, (size_t)n, hipMemcpyHostToDevice, r->h2d)) &&
                 ck(hipMemcpyAsync(am, t.absmax_m + b0, (size_t)nb * sizeof(float), hipMemcpyHostToDevice, r->h2d));
            if (two)
                ok = ok && ck(hipMemcpyAsync(v, t.v + off, (size_t)n, hipMemcpyHostToDevice, r->h2d)) &&
                     ck(hipMemcpyAsync(av, t.absmax_v + b0, (size_t)nb * sizeof(float), hipMemcpyHostToDevice,
                                       r->h2d));
            ok = ok && ck(hipEventRecord(r->in[slot], r->h2d)) && ck(hipStreamWaitEvent(s, r->in[slot], 0));
            if (!ok) return QB_EHIP;
            // the step of the page, on the caller's stream
            const size_t ps = pdt == QB_F32 ? 4 : 2, gs = gdt == QB_F32 ? 4 : 2;
            TensorDesc d{static_cast<char*>(t.p) + off * ps, static_cast<const char*>(t.g) + off * gs, m,
                         two ? v : nullptr, am, two ? av : nullptr, n, 0};
            hipError_t e = launch_optim8((int)hp->kind, d, nullptr, adamw_tiles(n, blocksize), blocksize, (int)pdt,
                                         (int)gdt, hs, nullptr, hp->v_code == QB_UDYN8, s);
            if (e != hipSuccess) return hip_status(e);
            // device to host after the step
            ok = ck(hipEventRecord(r->kern[slot], s)) && ck(hipStreamWaitEvent(r->d2h, r->kern[slot], 0)) &&
                 ck(hipMemcpyAsync(t.m + off, m, (size_t)n, hipMemcpyDeviceToHost, r->d2h)) &&
                 ck(hipMemcpyAsync(t.absmax_m + b0, am, (size_t)nb * sizeof(float), hipMemcpyDeviceToHost, r->d2h));
            if (two)
                ok = ok && ck(hipMemcpyAsync(t.v + off, v, (size_t)n, hipMemcpyDeviceToHost, r->d2h)) &&
                     ck(hipMemcpyAsync(t.absmax_v + b0, av, (size_t)nb * sizeof(float), hipMemcpyDeviceToHost,
                                       r->d2h));
            ok = ok && ck(hipEventRecord(r->out[slot], r->d2h));
            if (!ok) return QB_EHIP;
        }
    }
    // later work on `stream` waits for the last copy back
    if (!ck(hipEventRecord(r->done, r->d2h)) || !ck(hipStreamWaitEvent(s, r->done, 0))) return QB_EHIP;
    return QB_OK;
}

}  // extern "C"
