/*
 * Sanitizer driver for the CPU oracle (test infrastructure): calls every
 * oracle function on small, ragged inputs so that AddressSanitizer and
 * UndefinedBehaviorSanitizer see every code path.  Built and run by
 * tests/test_sanitizers.py with gcc -fsanitize=address,undefined; exits
 * non-zero on the first failing call (a sanitizer report aborts earlier).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_convert(const void* x, int xdt, void* y, int ydt, int64_t n);
int orc_dyn8_codebook(float* out);
int orc_udyn8_codebook(float* out);
int orc_nf4_codebook(float* out);
int orc_fp4_codebook(float* out);
int orc_linear_codebook(float* out);
int orc_encode(int code, const float* x, int64_t n, uint8_t* out);
int orc_quantize_blockwise(const void* x, int xdt, int64_t n, int code, int B, uint8_t* codes, float* absmax);
int orc_dequantize_blockwise(const uint8_t* codes, const float* scale, int code, int B, int64_t n, void* y, int ydt);
int orc_dq_quantize(const float* absmax, int64_t nb, float mu, int B2, uint8_t* c2, float* absmax2);
int orc_dq_decode(const uint8_t* c2, const float* absmax2, float mu, int B2, int64_t nb, float* a);
int orc_adamw32_step(float* p, const void* g, int gdt, int64_t n, float* m, float* v, double lr, double beta1,
                     double beta2, double eps, double wd, int step);
int orc_adamw8bit_step(float* p, const void* g, int gdt, int64_t n, uint8_t* cm, uint8_t* cv, float* am, float* av,
                       int B, double lr, double beta1, double beta2, double eps, double wd, int step);
int orc_optim32_step(int kind, const double* hp, int step, float* p, const void* g, int gdt, int64_t n, float* s1,
                     float* s2);
int orc_optim8bit_step(int kind, const double* hp, int step, float* p, const void* g, int gdt, int64_t n,
                       uint8_t* c1, uint8_t* c2, float* a1, float* a2, int B, int vcode);
int orc_quantize_custom(const void* x, int xdt, int64_t n, const float* cb, int B, uint8_t* codes, float* absmax);
int orc_dequantize_custom(const uint8_t* codes, const float* scale, const float* cb, int B, int64_t n, void* y,
                          int ydt);
int orc_quantile_averages(const void* x, int xdt, int64_t n, int C, double* A);
int orc_estimate_quantiles(const void* x, int xdt, int64_t n, int C, float* out);

#define CHECK(call)                                                                \
    do {                                                                           \
        if ((call) != 0) {                                                         \
            fprintf(stderr, "FAILED: %s (line %d)\n", #call, __LINE__);            \
            return 1;                                                              \
        }                                                                          \
    } while (0)

static uint32_t rng_state = 12345u;
static float frand(void) /* uniform in [-1, 1), xorshift */
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return (float)((double)rng_state / 2147483648.0 - 1.0);
}

int main(void)
{
    float cb[256];
    CHECK(orc_dyn8_codebook(cb));
    CHECK(orc_udyn8_codebook(cb));
    CHECK(orc_nf4_codebook(cb));
    CHECK(orc_fp4_codebook(cb));
    CHECK(orc_linear_codebook(cb));

    const int64_t sizes[] = {1, 2, 3, 63, 65, 257, 1000, 4097};
    const int blocks[] = {64, 256, 4096};
    for (int si = 0; si < 8; si++) {
        const int64_t n = sizes[si];
        float* x = malloc(sizeof(float) * n);
        uint16_t* h = malloc(sizeof(uint16_t) * n);
        float* y = malloc(sizeof(float) * n);
        uint8_t* codes = malloc(n);
        uint8_t* enc = malloc(n);
        for (int64_t i = 0; i < n; i++) x[i] = frand() * 0.02f * (i % 17 == 0 ? 50.0f : 1.0f);
        if (n > 5) x[3] = 0.0f, x[4] = -0.0f, x[5] = 1e-40f;          /* zeros and a subnormal */
        CHECK(orc_convert(x, 0, h, 1, n));                             /* binary32 -> fp16 */
        CHECK(orc_convert(h, 1, y, 0, n));
        CHECK(orc_convert(x, 0, h, 2, n));                             /* -> bf16 */
        for (int code = 0; code < 3; code++) {
            CHECK(orc_encode(code, x, n, enc));
            for (int bi = 0; bi < 3; bi++) {
                const int B = blocks[bi];
                const int64_t nb = (n + B - 1) / B;
                float* am = malloc(sizeof(float) * nb);
                for (int xdt = 0; xdt < 3; xdt++) {
                    const void* in = xdt == 0 ? (const void*)x : (const void*)h;
                    if (xdt == 1) CHECK(orc_convert(x, 0, h, 1, n));
                    if (xdt == 2) CHECK(orc_convert(x, 0, h, 2, n));
                    CHECK(orc_quantize_blockwise(in, xdt, n, code, B, codes, am));
                    for (int ydt = 0; ydt < 3; ydt++) CHECK(orc_dequantize_blockwise(codes, am, code, B, n, y, ydt));
                }
                uint8_t* c2 = malloc(nb);
                float* a2 = malloc(sizeof(float) * ((nb + 255) / 256));
                float* ad = malloc(sizeof(float) * nb);
                CHECK(orc_dq_quantize(am, nb, 0.01f, 256, c2, a2));
                CHECK(orc_dq_decode(c2, a2, 0.01f, 256, nb, ad));
                free(c2);
                free(a2);
                free(ad);
                free(am);
            }
        }
        /* user codes */
        CHECK(orc_linear_codebook(cb));
        {
            const int64_t nb = (n + 63) / 64;
            float* am = malloc(sizeof(float) * nb);
            CHECK(orc_quantize_custom(x, 0, n, cb, 64, codes, am));
            for (int ydt = 0; ydt < 3; ydt++) CHECK(orc_dequantize_custom(codes, am, cb, 64, n, y, ydt));
            free(am);
        }
        /* quantile estimation with ragged chunks */
        {
            double A[257];
            float q[256];
            CHECK(orc_quantile_averages(x, 0, n, 257, A));
            CHECK(orc_estimate_quantiles(x, 0, n, 300, q));
            CHECK(orc_estimate_quantiles(h, 2, n, 257, q));
        }
        /* optimizers: every kind, 8-bit and binary32 states, three steps */
        for (int kind = 0; kind < 7; kind++) {
            double hp[8] = {1e-3, 0.9, 0.999, 1e-8, 0.01, 0.0, 0.0, 1e-3};
            if (kind == 3) hp[3] = 0.0;                                  /* SGD: no eps */
            for (int vcode = 0; vcode < 4; vcode += 3) {
                if (vcode == 3 && !(kind == 0 || kind == 1 || kind == 4 || kind == 5)) continue;
                for (int bi = 0; bi < 3; bi++) {
                    const int B = blocks[bi];
                    const int64_t nb = (n + B - 1) / B;
                    float* p = malloc(sizeof(float) * n);
                    float* g = malloc(sizeof(float) * n);
                    uint8_t* c1 = malloc(n);
                    uint8_t* cc2 = malloc(n);
                    float* a1 = calloc(nb, sizeof(float));
                    float* a2 = calloc(nb, sizeof(float));
                    float* s1 = calloc(n, sizeof(float));
                    float* s2 = calloc(n, sizeof(float));
                    for (int64_t i = 0; i < n; i++) {
                        p[i] = x[i];
                        g[i] = frand() * 1e-3f;
                    }
                    memset(c1, kind == 4 && vcode == 3 ? 0 : 127, n);
                    memset(cc2, vcode == 3 ? 0 : 127, n);
                    for (int step = 1; step <= 3; step++) {
                        CHECK(orc_optim8bit_step(kind, hp, step, p, g, 0, n, c1, cc2, a1, a2, B, vcode));
                        CHECK(orc_optim32_step(kind, hp, step, p, g, 0, n, s1, s2));
                    }
                    free(p);
                    free(g);
                    free(c1);
                    free(cc2);
                    free(a1);
                    free(a2);
                    free(s1);
                    free(s2);
                }
            }
        }
        /* AdamW entry points with bf16 gradients */
        {
            const int64_t nb = (n + 2047) / 2048;
            float* p = malloc(sizeof(float) * n);
            float* m32 = calloc(n, sizeof(float));
            float* v32 = calloc(n, sizeof(float));
            uint8_t* cm = malloc(n);
            uint8_t* cv = malloc(n);
            float* am = calloc(nb, sizeof(float));
            float* av = calloc(nb, sizeof(float));
            memcpy(p, x, sizeof(float) * n);
            memset(cm, 127, n);
            memset(cv, 127, n);
            CHECK(orc_convert(x, 0, h, 2, n));
            for (int step = 1; step <= 3; step++) {
                CHECK(orc_adamw8bit_step(p, h, 2, n, cm, cv, am, av, 2048, 1e-3, 0.9, 0.999, 1e-8, 0.01, step));
                CHECK(orc_adamw32_step(p, h, 2, n, m32, v32, 1e-3, 0.9, 0.999, 1e-8, 0.01, step));
            }
            free(p);
            free(m32);
            free(v32);
            free(cm);
            free(cv);
            free(am);
            free(av);
        }
        free(x);
        free(h);
        free(y);
        free(codes);
        free(enc);
    }
    printf("oracle driver: all calls returned 0\n");
    return 0;
}
