/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for block-wise dynamic
 * quantization and the 8-bit AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, table or constant generator with
 * the HIP library.
 *
 * Conventions: IEEE binary32 arithmetic, round-to-nearest-even, every
 * operation rounded on its own (built with -ffp-contract=off -fno-fast-math),
 * denormals kept.  Inputs are finite.
 *
 * What is computed, and where the pages define it:
 *   - block-wise quantization: the tensor is cut into blocks of B elements,
 *     every block is scaled by its own absolute maximum and quantized on its
 *     own ("8-bit Optimizers via Block-wise Quantization" abstract, quoted on
 *     the page "Py之bitsandbytes：bitsandbytes的简介、安装、使用方法之详细攻略",
 *     section 2; the page "bitsandbytes深度解析", section 核心量化原理与实现机制);
 *   - the dynamic (non-linear) 8-bit code, precise for large and small
 *     magnitudes (same abstract; same page, section 1 lists quantile, linear and
 *     dynamic quantization);
 *   - the NF4 4-bit data type for normally distributed weights (page
 *     "Bitsandbytes" (Transformers docs, Turkish), section Normal Float 4 (NF4);
 *     page "Quantize 🤗 Transformers models", section Using NF4);
 *   - the FP4 4-bit data type (page "Quantize 🤗 Transformers models",
 *     section FP4 quantization), two 4-bit codes per byte (0.5 byte per
 *     parameter: page "bitsandbytes - Quantização de LLM", section Etapa 1);
 *   - nested (double) quantization of the per-block constants (page
 *     "Bitsandbytes", section İç içe nicelleştirme);
 *   - the 8-bit AdamW optimizer as a drop-in replacement of AdamW (page
 *     "bitsandbytes - Quantização de LLM", section Workflow 3; page
 *     "Py之bitsandbytes", section 使用8位优化器).
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that implements it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_DYN8 = 0, ORC_NF4 = 1, ORC_FP4 = 2, ORC_UDYN8 = 3 };
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* ------------------------------------------------------------------------ */
/* scalar conversions (written from the IEEE 754 binary16 / bfloat16 layout) */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* binary16 -> binary32, exact. */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t e = (h >> 10) & 0x1F;
    uint32_t m = h & 0x3FF;
    if (e == 0) {
        /* zero or subnormal: value = m * 2^-24 (exact in binary32) */
        float v = (float)m * (1.0f / 16777216.0f);
        return sign ? -v : v;
    }
    if (e == 31) return bits_to_f32(sign | 0x7F800000u | (m << 13));
    return bits_to_f32(sign | ((e - 15 + 127) << 23) | (m << 13));
}

/* bfloat16 -> binary32, exact: bfloat16 is the top half of a binary32. */
static float bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest even (finite inputs). */
static uint16_t f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint32_t keep = u >> 16, rest = u & 0xFFFF;
    if (rest > 0x8000 || (rest == 0x8000 && (keep & 1))) keep += 1;
    return (uint16_t)keep;
}

/* binary32 -> binary16, round to nearest even (finite inputs; overflow to inf). */
static uint16_t f32_to_f16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 31) << 15);
    float a = fabsf(f);
    if (a >= 65520.0f) return sign | 0x7C00; /* rounds to infinity */
    if (a < 6.103515625e-05f) {
        /* binary16 subnormal range: quantum 2^-24; a * 2^24 is exact */
        double q = (double)a * 16777216.0;     /* exact */
        double fl = floor(q);
        double r = q - fl;                     /* exact */
        uint32_t m = (uint32_t)fl;
        if (r > 0.5 || (r == 0.5 && (m & 1))) m += 1;
        return sign | (uint16_t)m;             /* m == 0x400 is the smallest normal */
    }
    int e = (int)((u >> 23) & 0xFF) - 127;     /* -14 .. 15 */
    uint32_t mant = (u & 0x7FFFFF) | 0x800000; /* 24 bits */
    uint32_t keep = mant >> 13, rest = mant & 0x1FFF;
    if (rest > 0x1000 || (rest == 0x1000 && (keep & 1))) keep += 1;
    uint32_t bits = ((uint32_t)(e + 15) << 10) + (keep - 0x400); /* carry moves into the exponent */
    return sign | (uint16_t)bits;
}

static float load_elem(const void* x, int dt, int64_t i)
{
    if (dt == ORC_F32) return ((const float*)x)[i];
    if (dt == ORC_F16) return f16_to_f32(((const uint16_t*)x)[i]);
    return bf16_to_f32(((const uint16_t*)x)[i]);
}

static void store_elem(void* y, int dt, int64_t i, float v)
{
    if (dt == ORC_F32) ((float*)y)[i] = v;
    else if (dt == ORC_F16) ((uint16_t*)y)[i] = f32_to_f16(v);
    else ((uint16_t*)y)[i] = f32_to_bf16(v);
}

/* exported for the tests that pin these conversions against a library routine */
float orc_f16_to_f32(uint16_t h) { return f16_to_f32(h); }

/* y[i] = x[i] converted from dtype xdt to ydt (widening exact; narrowing to
 * nearest even). */
int orc_convert(const void* x, int xdt, void* y, int ydt, int64_t n)
{
    for (int64_t i = 0; i < n; i++) store_elem(y, ydt, i, load_elem(x, xdt, i));
    return 0;
}
uint16_t orc_f32_to_f16(float f) { return f32_to_f16(f); }
uint16_t orc_f32_to_bf16(float f) { return f32_to_bf16(f); }

/* ------------------------------------------------------------------------ */
/* codebooks                                                                 */
/* ------------------------------------------------------------------------ */

static int cmp_float(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

/* Round a positive double to binary32; returns -1 if the double sits exactly
 * on a binary32 rounding tie (then double rounding could differ from rounding
 * the exact value once, and the caller must not trust it). */
static int round_to_f32_checked(double d, float* out)
{
    uint64_t u; memcpy(&u, &d, 8);
    if ((u & 0x1FFFFFFFull) == 0x10000000ull) return -1; /* exact halfway in binary32 */
    *out = (float)d;
    return 0;
}

/*
 * Dynamic 8-bit code (reading of "dynamic quantization ... precise for both
 * large and small magnitude values", abstract quoted on the page
 * "Py之bitsandbytes", section 2).  The reading taken is the dynamic tree code of
 * that paper: a sign, a decimal exponent and a linear fraction.  For decade
 * e = 0..6 there are 2^e linearly spaced magnitudes, the midpoints of 2^e equal
 * bins that split [0.1, 1] and are then scaled by 10^(e-6):
 *     v(e, j) = 10^(e-6) * (0.1 + 0.9 * (j + 1/2) / 2^e),   j = 0 .. 2^e - 1.
 * That gives 127 positive magnitudes; the code is their negatives, zero, the
 * magnitudes and +1.0, sorted ascending (256 entries; index 127 is 0.0 and 255
 * is +1.0).  Each value is the exact rational
 *     v(e, j) = (2^(e+1) + 18 j + 9) / (2^(e+1) * 10^(7-e))
 * rounded once to binary32.
 */
int orc_dyn8_codebook(float* out /* [256] */)
{
    float pos[127];
    int n = 0;
    for (int e = 0; e <= 6; e++) {
        for (int j = 0; j < (1 << e); j++) {
            int64_t pow10 = 1;
            for (int k = 0; k < 7 - e; k++) pow10 *= 10;
            double num = (double)((1 << (e + 1)) + 18 * j + 9);   /* exact integer */
            double den = (double)((int64_t)(1 << (e + 1)) * pow10); /* exact integer < 2^53 */
            float f;
            if (round_to_f32_checked(num / den, &f) != 0) return -1;
            pos[n++] = f;
        }
    }
    for (int i = 0; i < 127; i++) out[i] = -pos[126 - i];
    out[127] = 0.0f;
    for (int i = 0; i < 127; i++) out[128 + i] = pos[i];
    out[255] = 1.0f;
    qsort(out, 256, sizeof(float), cmp_float); /* already ascending; sorting states the rule */
    return 0;
}

/*
 * Unsigned dynamic 8-bit code, for a state that is never negative (v of Adam
 * and AdamW, the state of RMSprop).  Reading: the pages name only the signed
 * dynamic code; its plainest unsigned form spends the sign bit on one more
 * fraction bit, so each of the same seven decades holds twice as many linearly
 * spaced magnitudes, the midpoints of 2^(e+1) equal bins that split [0.1, 1],
 * scaled by 10^(e-6):
 *     u(e, j) = 10^(e-6) * (0.1 + 0.9 * (j + 1/2) / 2^(e+1)),   j = 0 .. 2^(e+1) - 1.
 * That gives 254 magnitudes; the code is 0, the magnitudes and +1.0, ascending
 * (index 0 is 0.0 and 255 is +1.0).  Each value is the exact rational
 *     u(e, j) = (2^(e+2) + 18 j + 9) / (2^(e+2) * 10^(7-e))
 * rounded once to binary32.
 */
int orc_udyn8_codebook(float* out /* [256] */)
{
    int n = 0;
    out[n++] = 0.0f;
    for (int e = 0; e <= 6; e++) {
        int64_t pow10 = 1;
        for (int k = 0; k < 7 - e; k++) pow10 *= 10;
        for (int j = 0; j < (2 << e); j++) {
            double num = (double)((4 << e) + 18 * j + 9);            /* exact integer */
            double den = (double)((int64_t)(4 << e) * pow10);        /* exact integer < 2^53 */
            float f;
            if (round_to_f32_checked(num / den, &f) != 0) return -1;
            out[n++] = f;
        }
    }
    out[n++] = 1.0f;                                   /* n == 256 */
    qsort(out, 256, sizeof(float), cmp_float);         /* already ascending */
    return 0;
}

/* Standard normal CDF from the complementary error function (libm, long double). */
static long double norm_cdf(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

/* Inverse standard normal CDF by bisection on norm_cdf: slow, obviously correct. */
static long double norm_ppf(long double p)
{
    long double lo = -12.0L, hi = 12.0L;
    for (int it = 0; it < 200; it++) {
        long double mid = 0.5L * (lo + hi);
        if (norm_cdf(mid) < p) lo = mid; else hi = mid;
    }
    return 0.5L * (lo + hi);
}

/*
 * NF4 (page "Bitsandbytes", section Normal Float 4 (NF4): a 4-bit type adapted
 * to weights initialised from a normal distribution, from the QLoRA paper).
 * Reading: the QLoRA construction from quantiles of N(0,1) with an exact zero.
 * With delta = (1/30 + 1/32)/2 and P = 1 - delta:
 *   8 positive values  ppf(1/2 + (P - 1/2) k/8), k = 1..8,
 *   7 negative values -ppf(1/2 + (P - 1/2) k/7), k = 1..7,
 *   and 0; all divided by ppf(P); 16 entries sorted ascending
 *   (index 0 = -1, index 7 = 0, index 15 = +1).
 */
int orc_nf4_codebook(float* out /* [16] */)
{
    long double delta = 0.5L * (1.0L / 30.0L + 1.0L / 32.0L);
    long double P = 1.0L - delta;
    long double scale = norm_ppf(P);
    int n = 0;
    for (int k = 7; k >= 1; k--) out[n++] = (float)(-norm_ppf(0.5L + (P - 0.5L) * k / 7.0L) / scale);
    out[n++] = 0.0f;
    for (int k = 1; k <= 8; k++) out[n++] = (float)(norm_ppf(0.5L + (P - 0.5L) * k / 8.0L) / scale);
    out[0] = -1.0f;  /* k = 7: -ppf(P)/ppf(P) */
    out[15] = 1.0f;  /* k = 8:  ppf(P)/ppf(P) */
    qsort(out, 16, sizeof(float), cmp_float);
    return 0;
}

/*
 * FP4 (page "Quantize 🤗 Transformers models", section FP4 quantization; the
 * pages only name the type).  Reading: the E2M1 minifloat, magnitudes
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}, divided by 6 so the largest is 1.  The 4-bit code
 * is sign-magnitude: code = s << 3 | k, k = index of the magnitude (also its
 * E2M1 bit pattern).  Table entries are indexed by code; code 8 (negative
 * zero) decodes to +0.0.
 */
static const double fp4_mag_numer[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int orc_fp4_codebook(float* out /* [16], indexed by code */)
{
    for (int k = 0; k < 8; k++) {
        float f;
        if (k == 0) f = 0.0f;
        else if (round_to_f32_checked(fp4_mag_numer[k] / 6.0, &f) != 0) return -1;
        out[k] = f;
        out[8 + k] = (k == 0) ? 0.0f : -f;
    }
    return 0;
}

/* Codebook in ascending order plus its size (FP4: the 8 magnitudes). */
static int sorted_table(int code, float* t)
{
    if (code == ORC_DYN8) { orc_dyn8_codebook(t); return 256; }
    if (code == ORC_UDYN8) { orc_udyn8_codebook(t); return 256; }
    if (code == ORC_NF4) { orc_nf4_codebook(t); return 16; }
    float f4[16];
    orc_fp4_codebook(f4);
    for (int k = 0; k < 8; k++) t[k] = f4[k];
    return 8;
}

/* ------------------------------------------------------------------------ */
/* nearest-code encoder                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Index of the entry of the ascending table cb[0..K) nearest to x under exact
 * arithmetic; a tie goes to the entry of smaller magnitude (toward zero).
 * Reading: the pages say only that values are mapped to the code; "nearest"
 * with ties toward zero is the plainest rule and keeps the encoder symmetric
 * under negation (between entries of equal magnitude, such as -a and a, a tie
 * goes to the upper one).  cb[k] <= x < cb[k+1] is found by bisection, then 2x
 * is compared with cb[k] + cb[k+1] in binary64, where both sides are exact for
 * the built-in codes (adjacent entries are within a factor of 64 of each
 * other, or one is 0).
 */
static int nearest_index(const float* cb, int K, float x)
{
    if (x <= cb[0]) return 0;
    if (x >= cb[K - 1]) return K - 1;
    int lo = 0, hi = K - 1; /* invariant: cb[lo] <= x < cb[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (cb[mid] <= x) lo = mid; else hi = mid;
    }
    double a = cb[lo], b = cb[hi];
    double sum = a + b;           /* exact for the built-in codes; for a user code the
                                     midpoint is read as computed in binary64 */
    double twice = 2.0 * (double)x;
    if (twice > sum) return hi;
    if (twice < sum) return lo;
    return (fabs(a) < fabs(b)) ? lo : hi;   /* equal magnitudes: the upper entry */
}

/* Encode one normalized value x in [-1, 1] with code `code`. */
static int encode(int code, const float* cb, int K, float x)
{
    if (code != ORC_FP4) return nearest_index(cb, K, x);
    int k = nearest_index(cb, K, fabsf(x));       /* nearest magnitude */
    return (x < 0.0f && k > 0) ? (8 | k) : k;      /* sign-magnitude; zero is +0 */
}

/* Exported for brute-force tests: encode an array of values. */
int orc_encode(int code, const float* x, int64_t n, uint8_t* out)
{
    float cb[256];
    int K = sorted_table(code, cb);
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)encode(code, cb, K, x[i]);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* block-wise quantize / dequantize                                          */
/* ------------------------------------------------------------------------ */

static int is_4bit(int code) { return code == ORC_NF4 || code == ORC_FP4; }

/*
 * quantize_blockwise: for block b = [bB, min(n, (b+1)B)):
 *   a_b = max |x_i|  (the block's absmax; a partial last block uses its tail);
 *   n_i = x_i / a_b  (IEEE binary32 division), or 0 when a_b == 0;
 *   c_i = nearest code of n_i.
 * 8-bit codes take one byte per element; 4-bit codes take one nibble, element
 * 2k in the high nibble and 2k+1 in the low nibble of byte k (reading: the pages
 * fix only two codes per byte); an odd n leaves the last low nibble 0.
 */
int orc_quantize_blockwise(const void* x, int xdt, int64_t n, int code, int B,
                           uint8_t* codes, float* absmax)
{
    float cb[256];
    int K = sorted_table(code, cb);
    int64_t nb = (n + B - 1) / B;
    if (is_4bit(code)) memset(codes, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * B, hi = lo + B < n ? lo + B : n;
        float a = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            float v = fabsf(load_elem(x, xdt, i));
            if (v > a) a = v;
        }
        absmax[b] = a;
        for (int64_t i = lo; i < hi; i++) {
            float nv = (a > 0.0f) ? load_elem(x, xdt, i) / a : 0.0f;
            int c = encode(code, cb, K, nv);
            if (is_4bit(code)) codes[i / 2] |= (uint8_t)((i % 2 == 0) ? (c << 4) : c);
            else codes[i] = (uint8_t)c;
        }
    }
    return 0;
}

/* Table indexed by code value as stored (DYN8/NF4: sorted index; FP4: s<<3|k). */
static void decode_table(int code, float* t)
{
    if (code == ORC_DYN8) orc_dyn8_codebook(t);
    else if (code == ORC_UDYN8) orc_udyn8_codebook(t);
    else if (code == ORC_NF4) orc_nf4_codebook(t);
    else orc_fp4_codebook(t);
}

/*
 * dequantize_blockwise: y_i = out_dtype(table[c_i] * s_b) with one binary32
 * multiply and one round-to-nearest-even conversion (the page "Bitsandbytes",
 * section on dequantizing; the compute dtype of the page "Quantize 🤗
 * Transformers models", section Change the compute dtype).  s_b is the
 * block's absmax.
 */
int orc_dequantize_blockwise(const uint8_t* codes, const float* scale, int code, int B,
                             int64_t n, void* y, int ydt)
{
    float t[256];
    decode_table(code, t);
    for (int64_t i = 0; i < n; i++) {
        int c = is_4bit(code) ? ((i % 2 == 0) ? (codes[i / 2] >> 4) : (codes[i / 2] & 15)) : codes[i];
        store_elem(y, ydt, i, t[c] * scale[i / B]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* double (nested) quantization of the absmax                                */
/* ------------------------------------------------------------------------ */

/*
 * Nested quantization (page "Bitsandbytes", section İç içe nicelleştirme: a
 * second quantization of the already quantized constants, saving about 0.4 bit
 * per parameter).  Reading: centre the fp32 absmax values a_j on their mean mu
 * (computed exactly and rounded once to binary32, by the caller), then quantize
 * d_j = a_j - mu (binary32 subtraction) block-wise with the dynamic 8-bit code
 * and block size B2.  Outputs: codes c2[nb], absmax2[ceil(nb/B2)].
 */
int orc_dq_quantize(const float* absmax, int64_t nb, float mu, int B2, uint8_t* c2, float* absmax2)
{
    float* d = (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
    if (!d) return -1;
    for (int64_t j = 0; j < nb; j++) d[j] = absmax[j] - mu;
    int rc = orc_quantize_blockwise(d, ORC_F32, nb, ORC_DYN8, B2, c2, absmax2);
    free(d);
    return rc;
}

/* Decoded absmax: a_j = dyn8[c2_j] * absmax2[j / B2] + mu, two rounded binary32 ops. */
int orc_dq_decode(const uint8_t* c2, const float* absmax2, float mu, int B2, int64_t nb, float* a)
{
    float t[256];
    orc_dyn8_codebook(t);
    for (int64_t j = 0; j < nb; j++) {
        float prod = t[c2[j]] * absmax2[j / B2];
        a[j] = prod + mu;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* AdamW with 8-bit block-wise dynamic state                                 */
/* ------------------------------------------------------------------------ */

/*
 * Host scalars of one AdamW step t >= 1 (reading: torch.optim.AdamW semantics,
 * because the pages present the 8-bit optimizer as a drop-in replacement for
 * AdamW with the same lr, betas and eps; page "bitsandbytes - Quantização de
 * LLM", section Workflow 3).  The hyperparameters are real numbers (binary64);
 * every scalar is computed in binary64 and rounded once to binary32:
 *   b1 = beta1, ob1 = 1 - beta1, b2 = beta2, ob2 = 1 - beta2,
 *   beta1^t and beta2^t by t repeated multiplications,
 *   s1 = lr / (1 - beta1^t), s2 = 1 / sqrt(1 - beta2^t), dec = 1 - lr*wd, eps.
 */
typedef struct { float b1, ob1, b2, ob2, s1, s2, dec, eps; } adam_scalars;

static adam_scalars adam_prepare(double lr, double beta1, double beta2, double eps, double wd, int step)
{
    double p1 = 1.0, p2 = 1.0;
    for (int i = 0; i < step; i++) { p1 *= beta1; p2 *= beta2; }
    adam_scalars s;
    s.b1 = (float)beta1;
    s.b2 = (float)beta2;
    s.ob1 = (float)(1.0 - beta1);
    s.ob2 = (float)(1.0 - beta2);
    s.s1 = (float)(lr / (1.0 - p1));
    s.s2 = (float)(1.0 / sqrt(1.0 - p2));
    s.dec = (float)(1.0 - lr * wd);
    s.eps = (float)eps;
    return s;
}

/*
 * One element of the update, binary32, each operation rounded:
 *   m' = b1*m + ob1*g
 *   v' = b2*v + ob2*(g*g)
 *   p' = p*dec - s1 * (m' / (sqrt(v')*s2 + eps))
 * (decoupled weight decay, bias correction, eps outside the square root).
 */
static void adam_elem(const adam_scalars* s, float g, float* p, float* m, float* v)
{
    float t1 = s->b1 * *m;
    float t2 = s->ob1 * g;
    float m1 = t1 + t2;
    float gg = g * g;
    float t3 = s->b2 * *v;
    float t4 = s->ob2 * gg;
    float v1 = t3 + t4;
    float den = sqrtf(v1) * s->s2 + s->eps;
    float upd = s->s1 * (m1 / den);
    float pd = *p * s->dec;
    *p = pd - upd;
    *m = m1;
    *v = v1;
}

/* AdamW with binary32 state (no quantization): pins the update against torch. */
int orc_adamw32_step(float* p, const void* g, int gdt, int64_t n, float* m, float* v,
                     double lr, double beta1, double beta2, double eps, double wd, int step)
{
    adam_scalars s = adam_prepare(lr, beta1, beta2, eps, wd, step);
    for (int64_t i = 0; i < n; i++) adam_elem(&s, load_elem(g, gdt, i), &p[i], &m[i], &v[i]);
    return 0;
}

/*
 * One 8-bit AdamW step.  Per block: dequantize both moments with the dynamic
 * code (m = dyn8[cm] * am, v = dyn8[cv] * av), apply the update above to every
 * element (the parameter update uses the unquantized m', v'), take the new block
 * absmax of m' and v', and quantize m' and v' back with the dynamic code
 * (same block-wise rule as orc_quantize_blockwise).  Initial state: codes of 0.0
 * (index 127) and absmax 0.
 */
int orc_adamw8bit_step(float* p, const void* g, int gdt, int64_t n, uint8_t* cm, uint8_t* cv,
                       float* am, float* av, int B,
                       double lr, double beta1, double beta2, double eps, double wd, int step)
{
    adam_scalars s = adam_prepare(lr, beta1, beta2, eps, wd, step);
    float cb[256];
    orc_dyn8_codebook(cb);
    float* mb = (float*)malloc(sizeof(float) * (size_t)B);
    float* vb = (float*)malloc(sizeof(float) * (size_t)B);
    if (!mb || !vb) { free(mb); free(vb); return -1; }
    int64_t nb = (n + B - 1) / B;
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * B, hi = lo + B < n ? lo + B : n;
        float a_m = 0.0f, a_v = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            float m = cb[cm[i]] * am[b];
            float v = cb[cv[i]] * av[b];
            adam_elem(&s, load_elem(g, gdt, i), &p[i], &m, &v);
            mb[i - lo] = m;
            vb[i - lo] = v;
            if (fabsf(m) > a_m) a_m = fabsf(m);
            if (fabsf(v) > a_v) a_v = fabsf(v);
        }
        am[b] = a_m;
        av[b] = a_v;
        for (int64_t i = lo; i < hi; i++) {
            float nm = (a_m > 0.0f) ? mb[i - lo] / a_m : 0.0f;
            float nv = (a_v > 0.0f) ? vb[i - lo] / a_v : 0.0f;
            cm[i] = (uint8_t)nearest_index(cb, 256, nm);
            cv[i] = (uint8_t)nearest_index(cb, 256, nv);
        }
    }
    free(mb);
    free(vb);
    return 0;
}

/* The host scalars, exported so tests can pin them against binary64 closed forms. */
int orc_adam_scalars(double lr, double beta1, double beta2, double eps, double wd, int step, float* out8)
{
    adam_scalars s = adam_prepare(lr, beta1, beta2, eps, wd, step);
    out8[0] = s.b1; out8[1] = s.ob1; out8[2] = s.b2; out8[3] = s.ob2;
    out8[4] = s.s1; out8[5] = s.s2; out8[6] = s.dec; out8[7] = s.eps;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* the sibling 8-bit optimizers                                              */
/* ------------------------------------------------------------------------ */

/*
 * The pages list 8-bit Adam, AdamW, SGD (with momentum), RMSprop and Lion
 * next to each other as drop-in replacements that keep their optimizer's
 * hyperparameters (page "bitsandbytes深度解析", section 优化器模块深度分析; page
 * "Py之bitsandbytes", sections 1 and 使用8位优化器).  Reading: each follows its
 * usual definition (torch.optim.Adam, SGD and RMSprop; Lion as published by
 * Chen et al., 2023), with every state tensor kept as block-wise dynamic 8-bit
 * codes exactly as for AdamW.  Binary32, each operation rounded on its own.
 *
 * hp[] = {lr, beta1, beta2, eps, weight_decay, dampening, nesterov, trust}; per kind:
 *   ORC_ADAMW    as orc_adamw8bit_step.
 *   ORC_ADAM     L2-coupled decay: gw = g + wd*p, then the Adam update with
 *                bias correction and no decoupled decay.  States m, v.
 *   ORC_LION     c = b1*m + (1-b1)*g; p' = p*(1 - lr*wd) - lr*sign(c);
 *                m' = b2*m + (1-b2)*g.  State m.
 *   ORC_SGD      gw = g + wd*p; buf = gw at step 1, else
 *                buf' = mu*buf + (1-dampening)*gw (mu = beta1);
 *                d = nesterov ? gw + mu*buf' : buf'; p' = p - lr*d.  State buf.
 *   ORC_RMSPROP  gw = g + wd*p; v' = al*v + (1-al)*gw*gw (al = beta2);
 *                p' = p - lr*(gw / (sqrt(v') + eps)).  State v.
 * The layer-wise kinds ORC_LAMB and ORC_LARS (hp[7] = trust coefficient) are
 * described at layerwise32 below.
 */
enum { ORC_ADAMW = 0, ORC_ADAM = 1, ORC_LION = 2, ORC_SGD = 3, ORC_RMSPROP = 4, ORC_LAMB = 5, ORC_LARS = 6 };

static int optim_states(int kind) { return (kind == ORC_ADAMW || kind == ORC_ADAM || kind == ORC_LAMB) ? 2 : 1; }
static int is_layerwise(int kind) { return kind == ORC_LAMB || kind == ORC_LARS; }

typedef struct {
    int kind, step, nesterov;
    adam_scalars a;                 /* Adam(W) scalars */
    float lr, wd, b1, ob1, b2, ob2, dec, omd, eps;
} optim_scalars;

static optim_scalars optim_prepare(int kind, const double* hp, int step)
{
    optim_scalars s;
    memset(&s, 0, sizeof s);
    s.kind = kind;
    s.step = step;
    s.nesterov = hp[6] != 0.0;
    /* LAMB takes Adam's direction without lr: s1 = 1/(1 - beta1^t) */
    s.a = adam_prepare(kind == ORC_LAMB ? 1.0 : hp[0], hp[1], hp[2], hp[3], kind == ORC_ADAMW ? hp[4] : 0.0, step);
    s.lr = (float)hp[0];
    s.wd = (float)hp[4];
    s.b1 = (float)hp[1];
    s.ob1 = (float)(1.0 - hp[1]);
    s.b2 = (float)hp[2];
    s.ob2 = (float)(1.0 - hp[2]);
    s.dec = (float)(1.0 - hp[0] * hp[4]);
    s.omd = (float)(1.0 - hp[5]);
    s.eps = (float)hp[3];
    return s;
}

/* One element: x1, x2 are the states (x2 unused by one-state kinds). */
static void optim_elem(const optim_scalars* s, float g, float* p, float* x1, float* x2)
{
    switch (s->kind) {
    case ORC_ADAMW:
        adam_elem(&s->a, g, p, x1, x2);
        break;
    case ORC_ADAM: {
        float t = s->wd * *p;
        float gw = g + t;
        adam_elem(&s->a, gw, p, x1, x2);   /* decoupled factor is 1: p*1 is exact */
        break;
    }
    case ORC_LION: {
        float t1 = s->b1 * *x1;
        float t2 = s->ob1 * g;
        float c = t1 + t2;
        float sg = c > 0.0f ? 1.0f : (c < 0.0f ? -1.0f : 0.0f);
        float pd = *p * s->dec;
        float u = s->lr * sg;
        *p = pd - u;
        float t3 = s->b2 * *x1;
        float t4 = s->ob2 * g;
        *x1 = t3 + t4;
        break;
    }
    case ORC_SGD: {
        float t = s->wd * *p;
        float gw = g + t;
        float buf;
        if (s->step == 1) {
            buf = gw;
        } else {
            float t1 = s->b1 * *x1;
            float t2 = s->omd * gw;
            buf = t1 + t2;
        }
        float d = buf;
        if (s->nesterov) {
            float t3 = s->b1 * buf;
            d = gw + t3;
        }
        float u = s->lr * d;
        *p = *p - u;
        *x1 = buf;
        break;
    }
    case ORC_RMSPROP: {
        float t = s->wd * *p;
        float gw = g + t;
        float t3 = s->b2 * *x1;
        float gg = gw * gw;
        float t4 = s->ob2 * gg;
        float v1 = t3 + t4;
        float den = sqrtf(v1) + s->eps;
        float q = gw / den;
        float u = s->lr * q;
        *p = *p - u;
        *x1 = v1;
        break;
    }
    }
}

static int optim_check(int kind, const double* hp, int step)
{
    if (kind < ORC_ADAMW || kind > ORC_LARS || step < 1) return -1;
    if (kind == ORC_SGD && !(hp[1] > 0.0)) return -1;   /* 8-bit SGD keeps a momentum state */
    if (kind == ORC_LARS && !(hp[7] > 0.0)) return -1;  /* LARS needs a trust coefficient */
    return 0;
}

/*
 * The layer-wise kinds.  The pages list 8-bit LARS and LAMB among the 8-bit
 * optimizers (page "Py之bitsandbytes", section 1: 8-bit optimizers) and give
 * no formulas.  Reading: their published definitions, one call being one layer
 * (the norms run over the whole tensor) -- LARS as You, Gitman and Ginsburg
 * (2017) define it, with the local rate inside the momentum; LAMB as You et al.
 * (2019) define it, with bias correction and phi the identity.  The norms and
 * the ratio are binary64 (squares of binary32 values are exact in binary64;
 * the sums run in index order), and the ratio reaches the binary32 update as
 * one scalar S = (float)(lr * ratio); a zero norm makes the ratio 1:
 *   ORC_LAMB  states m, v:  m' = b1*m + (1-b1)*g,  v' = b2*v + (1-b2)*g*g,
 *             r = s1*(m' / (sqrt(v')*s2 + eps)) with s1 = 1/(1-b1^t) and
 *             s2 = 1/sqrt(1-b2^t) (adam_elem's order without lr),
 *             u = r + wd*p;  ratio = |p| / |u|;  p' = p - S*u.
 *   ORC_LARS  state buf (mu = beta1, eta = trust coefficient):
 *             ratio = eta*|p| / (|g| + wd*|p|);  gw = g + wd*p;
 *             buf' = mu*buf + S*gw;  p' = p - buf'.
 * x1, x2: binary32 states, updated in place.
 */
static int layerwise32(int kind, const double* hp, const optim_scalars* s, float* p, const void* g, int gdt,
                       int64_t n, float* x1, float* x2)
{
    double sp = 0.0, sq = 0.0;           /* |p|^2 and |u|^2 (LAMB) or |g|^2 (LARS) */
    float* u = NULL;
    if (kind == ORC_LAMB) {
        u = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
        if (!u) return -1;
        for (int64_t i = 0; i < n; i++) {
            float gi = load_elem(g, gdt, i);
            float t1 = s->a.b1 * x1[i];
            float t2 = s->a.ob1 * gi;
            float m1 = t1 + t2;
            float gg = gi * gi;
            float t3 = s->a.b2 * x2[i];
            float t4 = s->a.ob2 * gg;
            float v1 = t3 + t4;
            float den = sqrtf(v1) * s->a.s2 + s->a.eps;
            float r = s->a.s1 * (m1 / den);
            float t = s->wd * p[i];
            u[i] = r + t;
            x1[i] = m1;
            x2[i] = v1;
            sp += (double)p[i] * (double)p[i];
            sq += (double)u[i] * (double)u[i];
        }
    } else {
        for (int64_t i = 0; i < n; i++) {
            double gi = (double)load_elem(g, gdt, i);
            sp += (double)p[i] * (double)p[i];
            sq += gi * gi;
        }
    }
    double pn = sqrt(sp), qn = sqrt(sq);
    double ratio = 1.0;
    if (pn > 0.0 && qn > 0.0) ratio = (kind == ORC_LAMB) ? pn / qn : (hp[7] * pn) / (qn + hp[4] * pn);
    float S = (float)(hp[0] * ratio);
    for (int64_t i = 0; i < n; i++) {
        if (kind == ORC_LAMB) {
            float t = S * u[i];
            p[i] = p[i] - t;
        } else {
            float gi = load_elem(g, gdt, i);
            float t = s->wd * p[i];
            float gw = gi + t;
            float t1 = s->b1 * x1[i];
            float t2 = S * gw;
            float buf = t1 + t2;
            p[i] = p[i] - buf;
            x1[i] = buf;
        }
    }
    free(u);
    return 0;
}

/* Any kind with binary32 states (no quantization): pins the update rules. */
int orc_optim32_step(int kind, const double* hp, int step, float* p, const void* g, int gdt, int64_t n,
                     float* x1, float* x2)
{
    if (optim_check(kind, hp, step) != 0) return -1;
    optim_scalars s = optim_prepare(kind, hp, step);
    if (is_layerwise(kind)) return layerwise32(kind, hp, &s, p, g, gdt, n, x1, x2);
    float dummy = 0.0f;
    for (int64_t i = 0; i < n; i++)
        optim_elem(&s, load_elem(g, gdt, i), &p[i], &x1[i], optim_states(kind) == 2 ? &x2[i] : &dummy);
    return 0;
}

/*
 * Any kind with block-wise dynamic 8-bit states (c1/a1, and c2/a2 for the
 * two-state kinds; NULL otherwise): per block, decode the states, update every
 * element, take each state's new block absmax, encode again.  vcode is the
 * code of the state that is never negative (v of the two-state kinds, the
 * state of RMSprop): ORC_DYN8, or ORC_UDYN8 (the unsigned code above); every
 * other state takes ORC_DYN8.  A kind with no such state must pass ORC_DYN8.
 */
int orc_optim8bit_step(int kind, const double* hp, int step, float* p, const void* g, int gdt, int64_t n,
                       uint8_t* c1, uint8_t* c2, float* a1, float* a2, int B, int vcode)
{
    if (optim_check(kind, hp, step) != 0) return -1;
    const int two = optim_states(kind) == 2;
    if (vcode != ORC_DYN8 && vcode != ORC_UDYN8) return -1;
    if (vcode == ORC_UDYN8 && !two && kind != ORC_RMSPROP) return -1;
    const int code1 = kind == ORC_RMSPROP ? vcode : ORC_DYN8, code2 = vcode;
    optim_scalars s = optim_prepare(kind, hp, step);
    if (is_layerwise(kind)) {
        /* the norms span the whole tensor: decode every block, take the
         * binary32 step, quantize every block again */
        size_t bytes = sizeof(float) * (size_t)(n > 0 ? n : 1);
        float* x = (float*)malloc(bytes);
        float* y = (float*)malloc(bytes);
        int rc = -1;
        if (x && y) {
            orc_dequantize_blockwise(c1, a1, code1, B, n, x, ORC_F32);
            if (two) orc_dequantize_blockwise(c2, a2, code2, B, n, y, ORC_F32);
            rc = layerwise32(kind, hp, &s, p, g, gdt, n, x, two ? y : NULL);
            if (rc == 0) rc = orc_quantize_blockwise(x, ORC_F32, n, code1, B, c1, a1);
            if (rc == 0 && two) rc = orc_quantize_blockwise(y, ORC_F32, n, code2, B, c2, a2);
        }
        free(x);
        free(y);
        return rc;
    }
    float cb1[256], cb2[256];
    decode_table(code1, cb1);
    decode_table(code2, cb2);
    float* xb = (float*)malloc(sizeof(float) * (size_t)B);
    float* yb = (float*)malloc(sizeof(float) * (size_t)B);
    if (!xb || !yb) { free(xb); free(yb); return -1; }
    int64_t nb = (n + B - 1) / B;
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * B, hi = lo + B < n ? lo + B : n;
        float m1 = 0.0f, m2 = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            float x = cb1[c1[i]] * a1[b];
            float y = two ? cb2[c2[i]] * a2[b] : 0.0f;
            optim_elem(&s, load_elem(g, gdt, i), &p[i], &x, &y);
            xb[i - lo] = x;
            yb[i - lo] = y;
            if (fabsf(x) > m1) m1 = fabsf(x);
            if (fabsf(y) > m2) m2 = fabsf(y);
        }
        a1[b] = m1;
        if (two) a2[b] = m2;
        for (int64_t i = lo; i < hi; i++) {
            c1[i] = (uint8_t)nearest_index(cb1, 256, m1 > 0.0f ? xb[i - lo] / m1 : 0.0f);
            if (two) c2[i] = (uint8_t)nearest_index(cb2, 256, m2 > 0.0f ? yb[i - lo] / m2 : 0.0f);
        }
    }
    free(xb);
    free(yb);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* user codes: the linear code and estimated quantile codes                  */
/* ------------------------------------------------------------------------ */

/*
 * The pages list three 8-bit quantization types: quantile, linear and dynamic
 * (page "Py之bitsandbytes", section 1), and a fast quantile estimation.
 *
 * Linear code (reading: the symmetric 8-bit integer grid scaled by 1/127):
 * entries k/127 for k = -128 .. 127, ascending (index 128 is 0.0, 255 is 1.0).
 */
int orc_linear_codebook(float* out /* [256] */)
{
    for (int k = -128; k <= 127; k++) out[k + 128] = (float)((double)k / 127.0);
    return 0;
}

/* Block-wise quantize / dequantize with a user code (256 ascending entries). */
int orc_quantize_custom(const void* x, int xdt, int64_t n, const float* cb, int B, uint8_t* codes, float* absmax)
{
    for (int k = 0; k + 1 < 256; k++)
        if (!(cb[k] <= cb[k + 1]) || !isfinite(cb[k]) || !isfinite(cb[k + 1])) return -1;
    int64_t nb = (n + B - 1) / B;
    for (int64_t b = 0; b < nb; b++) {
        int64_t lo = b * B, hi = lo + B < n ? lo + B : n;
        float a = 0.0f;
        for (int64_t i = lo; i < hi; i++) {
            float v = fabsf(load_elem(x, xdt, i));
            if (v > a) a = v;
        }
        absmax[b] = a;
        for (int64_t i = lo; i < hi; i++) {
            float nv = (a > 0.0f) ? load_elem(x, xdt, i) / a : 0.0f;
            codes[i] = (uint8_t)nearest_index(cb, 256, nv);
        }
    }
    return 0;
}

int orc_dequantize_custom(const uint8_t* codes, const float* scale, const float* cb, int B, int64_t n, void* y,
                          int ydt)
{
    for (int64_t i = 0; i < n; i++) store_elem(y, ydt, i, cb[codes[i]] * scale[i / B]);
    return 0;
}

static int cmp_float_asc(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

/*
 * Exact sums of binary32 values.  A finite binary32 f is m * 2^(e - 150) with
 * an integer m < 2^24 and e = max(biased exponent, 1); exponent bin e - 1
 * accumulates the signed m in int64 (exact for fewer than 2^39 values), so
 * the sum is the exact integer N = sum_b bin[b] * 2^b, in units of 2^-149.
 * N is held in two's complement in 16 little-endian 32-bit limbs (|N| < 2^320
 * for the counts allowed here).
 */
enum { BIG_LIMBS = 16 };

static void f32_bin_add(int64_t* bins /* [254] */, float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t e = (u >> 23) & 0xFF;
    int64_t m = (int64_t)((u & 0x7FFFFF) | (e ? 0x800000u : 0u));
    bins[(e ? e : 1) - 1] += (u >> 31) ? -m : m;
}

/* big += v * 2^sh, v signed (two's complement add of the sign-extended value) */
static void big_add_shifted(uint32_t* big, int64_t v, int sh)
{
    uint32_t add[BIG_LIMBS];
    uint64_t uv = (uint64_t)v;
    uint32_t ext = v < 0 ? 0xFFFFFFFFu : 0u;
    for (int k = 0; k < BIG_LIMBS; k++) add[k] = ext;
    /* place the 64-bit value at bit sh; limbs above it keep the sign extension */
    int q = sh / 32, r = sh % 32;
    for (int k = 0; k < q && k < BIG_LIMBS; k++) add[k] = 0;
    uint32_t w0 = (uint32_t)uv, w1 = (uint32_t)(uv >> 32);
    uint32_t parts[3];
    parts[0] = w0 << r;
    parts[1] = r ? ((w1 << r) | (w0 >> (32 - r))) : w1;
    parts[2] = r ? ((ext << r) | (w1 >> (32 - r))) : ext;
    for (int k = 0; k < 3 && q + k < BIG_LIMBS; k++) add[q + k] = parts[k];
    uint64_t carry = 0;
    for (int k = 0; k < BIG_LIMBS; k++) {
        uint64_t s = (uint64_t)big[k] + add[k] + carry;
        big[k] = (uint32_t)s;
        carry = s >> 32;
    }
}

/*
 * The binary64 nearest (ties to even) to N * 2^-149 / d for the exact integer
 * N (two's complement, destroyed) and 0 < d < 2^32.  |N| * 2^96 is divided by
 * d in long division; the quotient Q has at least 65 bits when N != 0, so its
 * top 53 bits, the next bit and a sticky bit (lower bits of Q, remainder)
 * round it, and the result is (rounded Q) * 2^(shift - 245) in the normal
 * range of binary64.
 */
static double big_div_rn64(uint32_t* big, uint32_t d)
{
    int neg = (big[BIG_LIMBS - 1] >> 31) != 0;
    if (neg) {                                  /* magnitude: two's complement negation */
        uint64_t carry = 1;
        for (int k = 0; k < BIG_LIMBS; k++) {
            uint64_t s = (uint64_t)(uint32_t)~big[k] + carry;
            big[k] = (uint32_t)s;
            carry = s >> 32;
        }
    }
    uint32_t num[BIG_LIMBS + 3], quo[BIG_LIMBS + 3];
    for (int k = 0; k < 3; k++) num[k] = 0;             /* times 2^96 */
    for (int k = 0; k < BIG_LIMBS; k++) num[k + 3] = big[k];
    uint64_t rem = 0;
    for (int k = BIG_LIMBS + 2; k >= 0; k--) {
        uint64_t cur = (rem << 32) | num[k];
        quo[k] = (uint32_t)(cur / d);
        rem = cur % d;
    }
    int top = BIG_LIMBS + 2;
    while (top >= 0 && quo[top] == 0) top--;
    if (top < 0) return 0.0;
    int hb = 31;
    while (!((quo[top] >> hb) & 1u)) hb--;
    int bitlen = top * 32 + hb + 1;                     /* >= 65 */
    int shift = bitlen - 53;
    uint64_t sig = 0;
    for (int b = bitlen - 1; b >= shift; b--) sig = (sig << 1) | ((quo[b / 32] >> (b % 32)) & 1u);
    int guard = (quo[(shift - 1) / 32] >> ((shift - 1) % 32)) & 1u;
    int sticky = rem != 0;
    for (int b = 0; b < shift - 1 && !sticky; b++) sticky = (quo[b / 32] >> (b % 32)) & 1u;
    if (guard && (sticky || (sig & 1u))) {
        sig += 1;
        if (sig == (1ull << 53)) {
            sig >>= 1;
            shift += 1;
        }
    }
    double r = ldexp((double)sig, shift - 245);
    return neg ? -r : r;
}

/*
 * Quantile estimates of the data (reading of the pages' fast quantile
 * estimation): x is split into chunks of C consecutive values (the last may
 * be shorter), each chunk is sorted on its own, and the chunks' order
 * statistics are averaged:
 *   E_j(chunk of L sorted values s) = s[floor(j * L / 257)],  j = 0..256,
 *   A_j = the exact arithmetic mean of E_j over the chunks, rounded once to
 *         the nearest binary64 (ties to even), so it does not depend on the
 *         order in which the chunks are added.
 * A negative zero in x counts as +0.
 */
int orc_quantile_averages(const void* x, int xdt, int64_t n, int C, double* A /* [257] */)
{
    if (n < 1 || C < 257) return -1;
    int64_t nch = (n + C - 1) / C;
    if (nch >= ((int64_t)1 << 32)) return -1;
    int64_t* bins = (int64_t*)calloc((size_t)257 * 254, sizeof(int64_t));
    float* s = (float*)malloc(sizeof(float) * (size_t)C);
    if (!bins || !s) {
        free(bins);
        free(s);
        return -1;
    }
    for (int64_t c = 0; c < nch; c++) {
        int64_t lo = c * C, hi = lo + C < n ? lo + C : n;
        int L = (int)(hi - lo);
        for (int i = 0; i < L; i++) {
            float v = load_elem(x, xdt, lo + i);
            s[i] = v == 0.0f ? 0.0f : v;       /* -0 counts as +0: the sort orders numbers */
        }
        qsort(s, (size_t)L, sizeof(float), cmp_float_asc);
        for (int j = 0; j < 257; j++) f32_bin_add(bins + (size_t)j * 254, s[(int64_t)j * L / 257]);
    }
    free(s);
    for (int j = 0; j < 257; j++) {
        uint32_t big[BIG_LIMBS];
        memset(big, 0, sizeof(big));
        for (int b = 0; b < 254; b++)
            if (bins[(size_t)j * 254 + b]) big_add_shifted(big, bins[(size_t)j * 254 + b], b);
        A[j] = big_div_rn64(big, (uint32_t)nch);
    }
    free(bins);
    return 0;
}

/*
 * Quantile code estimated from data (reading of the pages' quantile
 * quantization and fast quantile estimation): the code entries are the
 * midpoints of adjacent quantile estimates A_j (orc_quantile_averages, at
 * probabilities j/257), normalized so that the largest magnitude is 1:
 *   q_i = (A_i + A_{i+1}) / 2,  i = 0..255                           (binary64),
 *   code_i = binary32(q_i / max_k |q_k|)   (all 0 when max_k |q_k| = 0).
 * The entries come out ascending (A is non-decreasing); equal neighbours are
 * possible.
 */
int orc_estimate_quantiles(const void* x, int xdt, int64_t n, int C, float* out /* [256] */)
{
    double A[257], q[256], m = 0.0;
    int rc = orc_quantile_averages(x, xdt, n, C, A);
    if (rc) return rc;
    for (int i = 0; i < 256; i++) {
        q[i] = (A[i] + A[i + 1]) * 0.5;
        if (fabs(q[i]) > m) m = fabs(q[i]);
    }
    for (int i = 0; i < 256; i++) out[i] = m > 0.0 ? (float)(q[i] / m) : 0.0f;
    return 0;
}
