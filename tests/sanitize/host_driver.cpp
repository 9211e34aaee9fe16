// Sanitizer driver for libqb's host code (test infrastructure): the exact
// table builder (qb_tables.cpp) and every C-ABI entry point's argument checks
// and host arithmetic (qb_api.cpp), built with -fsanitize=address,undefined
// against host_stubs.cpp instead of the HIP sources.  Pointers passed as
// "device" buffers are fake, 16-byte aligned addresses that are never
// dereferenced: every call must stop at a check (an error status) or at
// QB_EINIT (no device tables) before any copy or launch.  Exits non-zero on
// the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "qb.h"

static int failures = 0;
#define EXPECT(call, want)                                                                          \
    do {                                                                                            \
        const int got_ = (int)(call);                                                               \
        if (got_ != (int)(want)) {                                                                  \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_,   \
                         (int)(want));                                                              \
            ++failures;                                                                             \
        }                                                                                           \
    } while (0)

int main()
{
    // fake, aligned device addresses (never dereferenced)
    char* const D = reinterpret_cast<char*>(uintptr_t(1) << 40);
    void* const A = D;
    float* const F = reinterpret_cast<float*>(D + 4096);
    uint8_t* const U = reinterpret_cast<uint8_t*>(D + 8192);

    // host-side tables: every code, every table the kernels use
    float cb[256];
    for (int c = 0; c < 4; ++c) {
        const int k = qb_codebook((qb_code)c, cb);
        if (k != (c == 0 || c == 3 ? 256 : 16)) ++failures;
        for (int i = 1; i < k && (c != 2); ++i)
            if (!(cb[i - 1] < cb[i])) ++failures;          // sorted (FP4 is indexed by sign-magnitude code)
        const int need = qb_encoder_table((qb_code)c, nullptr, 0);
        std::vector<uint32_t> t(need > 0 ? 2 * (size_t)need : 2);   // two words per entry
        EXPECT(qb_encoder_table((qb_code)c, t.data(), need), need);
    }
    EXPECT(qb_codebook((qb_code)7, cb), -1);
    EXPECT(qb_linear_code(cb), 256);
    for (int s = -1; s < 9; ++s)
        if (!qb_status_string((qb_status)s)) ++failures;

    // workspace sizes
    for (int64_t n : {int64_t(0), int64_t(1), int64_t(4095), int64_t(1) << 33}) {
        (void)qb_dq_workspace_bytes(n, 64);
        (void)qb_quantile_workspace_bytes(n);
    }
    for (int c : {0, 1, 7, 291, 4096, 5000}) (void)qb_multi_tensor_workspace_bytes(c);
    EXPECT(qb_paged_workspace_bytes(2048 * 8, 2048) > 0, 1);
    EXPECT(qb_paged_workspace_bytes(100, 2048), 0);
    (void)qb_code_table_bytes();

    // quantize / dequantize / normalize
    qb_dq dq{U, F, F, 256, A, 1 << 20};
    EXPECT(qb_quantize(A, QB_F32, 0, QB_DYN8, 2048, U, F, nullptr, nullptr), QB_OK);
    EXPECT(qb_quantize(A, QB_F32, 1000, QB_DYN8, 100, U, F, nullptr, nullptr), QB_EINVAL);
    EXPECT(qb_quantize(A, QB_F32, 1000, QB_UDYN8, 2048, U, F, nullptr, nullptr), QB_EINVAL);
    EXPECT(qb_quantize(D + 4, QB_F32, 1000, QB_DYN8, 2048, U, F, nullptr, nullptr), QB_EALIGN);
    EXPECT(qb_quantize(A, QB_F32, 1000, QB_DYN8, 2048, U, F, nullptr, nullptr), QB_EINIT);
    EXPECT(qb_quantize(A, QB_F16, 1000, QB_NF4, 64, U, nullptr, &dq, nullptr), QB_EINIT);
    EXPECT(qb_dequantize(U, F, nullptr, QB_FP4, 64, 1000, A, QB_BF16, nullptr), QB_EINIT);
    EXPECT(qb_dequantize(U, nullptr, nullptr, QB_FP4, 64, 1000, A, QB_BF16, nullptr), QB_EINVAL);
    EXPECT(qb_normalize(A, QB_F32, 100, F, 0, F, nullptr), QB_EINVAL);
    EXPECT(qb_normalize(A, QB_F32, 100, F, 64, F, nullptr), QB_EHIP);     // reaches the (stub) launcher

    // grouped calls
    qb_quant_tensor qt[3] = {{A, U, F, nullptr, nullptr, nullptr, 5000}, {A, U, F, nullptr, nullptr, nullptr, 0},
                             {A, U, F, nullptr, nullptr, nullptr, 70000}};
    const size_t qws = qb_multi_tensor_quantize_workspace_bytes(qt, 3, 64);
    EXPECT(qb_multi_tensor_quantize(qt, 3, QB_F16, QB_NF4, 64, 256, A, qws, nullptr), QB_EINIT);
    EXPECT(qb_multi_tensor_quantize(qt, 3, QB_F16, QB_NF4, 64, 256, A, 0, nullptr), QB_EWORKSPACE);
    qb_dequant_tensor dt[2] = {{U, F, nullptr, nullptr, nullptr, A, 5000}, {U, F, nullptr, nullptr, nullptr, A, 9}};
    EXPECT(qb_multi_tensor_dequantize(dt, 2, QB_NF4, 64, 256, QB_BF16, A, qb_multi_tensor_workspace_bytes(2),
                                      nullptr),
           QB_EINIT);

    // optimizer steps
    qb_adamw_hparams hp{1e-3, 0.9, 0.999, 1e-8, 0.01, 1};
    EXPECT(qb_adamw8bit_step(F, A, QB_BF16, 4097, U, U, F, F, 2048, &hp, nullptr), QB_EINIT);
    EXPECT(qb_adamw8bit_step(F, F, QB_BF16, 4097, U, U, F, F, 2048, &hp, nullptr), QB_EINVAL);   // p aliases g
    qb_adamw_hparams bad = hp;
    bad.beta2 = 1.0;
    EXPECT(qb_adamw8bit_step(F, A, QB_BF16, 4097, U, U, F, F, 2048, &bad, nullptr), QB_EINVAL);
    std::vector<qb_tensor> ts;
    for (int i = 0; i < 300; ++i) ts.push_back(qb_tensor{F, A, U, U, F, F, (int64_t)(i * 37 % 5001)});
    const size_t mws = qb_multi_tensor_workspace_bytes(300);
    EXPECT(qb_multi_tensor_step(ts.data(), 300, QB_BF16, 256, &hp, A, mws, nullptr), QB_EINIT);
    EXPECT(qb_multi_tensor_step(ts.data(), 300, QB_BF16, 256, &hp, A, mws - 1, nullptr), QB_EWORKSPACE);
    EXPECT(qb_multi_tensor_step_noalloc(ts.data(), 300, QB_BF16, 256, &hp, nullptr), QB_EHIP);  // no scratch
    EXPECT(qb_multi_tensor_step_noalloc(ts.data(), 4097, QB_BF16, 256, &hp, nullptr), QB_EWORKSPACE);
    for (int kind = 0; kind < 7; ++kind) {
        qb_optim_hparams o{};
        o.kind = (qb_optimizer)kind;
        o.lr = 1e-3;
        o.beta1 = 0.9;
        o.beta2 = 0.99;
        o.eps = 1e-8;
        o.weight_decay = 0.01;
        o.step = 3;
        o.trust_coefficient = 1e-3;
        const size_t ows = qb_optimizer_workspace_bytes(&o, ts.data(), 300, 2048);
        EXPECT(qb_multi_tensor_optimizer_step(&o, ts.data(), 300, QB_F32, QB_BF16, 2048, A, ows, nullptr), QB_EINIT);
        if (kind != 5 && kind != 6)
            EXPECT(qb_optimizer8bit_step(&o, F, QB_F32, A, QB_BF16, 70001, U, U, F, F, 2048, nullptr), QB_EINIT);
        // paged: the states are not pinned host memory
        EXPECT(qb_paged_optimizer_step(&o, ts.data(), 300, QB_F32, QB_BF16, 2048, 2048 * 4, A,
                                       qb_paged_workspace_bytes(2048 * 4, 2048), nullptr),
               (kind == 5 || kind == 6) ? QB_EUNSUPPORTED : QB_EINVAL);
    }

    // user codes (only the rejecting paths of qb_prepare_code: a valid call copies to the table)
    float vals[256];
    for (int k = 0; k < 256; ++k) vals[k] = (float)k / 255.0f;
    vals[7] = vals[9];
    EXPECT(qb_prepare_code(vals, A, nullptr), QB_EINVAL);
    EXPECT(qb_estimate_quantiles(A, QB_F32, 100000, A, nullptr, A, qb_quantile_workspace_bytes(100000), nullptr),
           QB_EHIP);
    EXPECT(qb_quantize_code(A, QB_F32, 1000, A, 256, U, F, nullptr), QB_EHIP);      // the (stub) launcher
    EXPECT(qb_dequantize_code(U, F, A, 256, 1000, A, QB_F32, nullptr), QB_EHIP);

    // fused 4-bit product
    EXPECT(qb_dequant_matmul(A, QB_BF16, 16, 4096, U, F, nullptr, QB_NF4, 64, 4096, A, nullptr), QB_EINIT);
    EXPECT(qb_dequant_matmul(A, QB_BF16, 16, 4001, U, F, nullptr, QB_NF4, 64, 4096, A, nullptr), QB_EINVAL);
    // grouped: the full group of eight (one empty, skipped), then one too many
    qb_matmul_weight wts[QB_MATMUL_GROUP_MAX + 1];
    for (int i = 0; i <= QB_MATMUL_GROUP_MAX; ++i) wts[i] = qb_matmul_weight{U, F, nullptr, nullptr, nullptr, A, 64 + i};
    wts[3].N = 0;
    wts[3].codes = nullptr;
    EXPECT(qb_dequant_matmul_grouped(A, QB_BF16, 4, 4096, wts, QB_MATMUL_GROUP_MAX, QB_NF4, 64, 256, nullptr), QB_EINIT);
    EXPECT(qb_dequant_matmul_grouped(A, QB_BF16, 4, 4096, wts, QB_MATMUL_GROUP_MAX + 1, QB_NF4, 64, 256, nullptr),
           QB_EINVAL);

    if (failures) {
        std::fprintf(stderr, "host driver: %d unexpected results\n", failures);
        return 1;
    }
    std::printf("host driver: every call returned the expected status\n");
    return 0;
}
