/*
 * qb.h -- C ABI of libqb: block-wise dynamic quantization, nested quantization
 * of the block constants, the fused 8-bit AdamW step and its sibling 8-bit
 * optimizers (with paged states), user codes, and the product of a 4-bit
 * layer, for AMD Instinct MI355X (gfx950).
 *
 * The method: a tensor is cut into blocks of `blocksize` consecutive elements;
 * every block is scaled by its own absolute maximum and each scaled value is
 * replaced by the index of the nearest entry of a fixed code, so blocks are
 * quantized independently and in parallel (abstract of "8-bit Optimizers via
 * Block-wise Quantization", quoted on the page "Py之bitsandbytes：bitsandbytes的
 * 简介、安装、使用方法之详细攻略", section 2; page "bitsandbytes深度解析",
 * section 核心量化原理与实现机制).
 *
 * Codes (QB_DYN8, QB_NF4, QB_FP4, QB_UDYN8) -- see qb_codebook() for the exact
 * tables:
 *   QB_DYN8  256-entry signed dynamic code (decimal exponent + linear fraction),
 *            one byte per element; index 127 is 0.0, 255 is +1.0.
 *   QB_UDYN8 256-entry unsigned dynamic code for an optimizer state that is
 *            never negative (see qb_optim_hparams.v_code): the sign bit of
 *            QB_DYN8 spent on one more fraction bit, so each of the same seven
 *            decades holds twice as many values; index 0 is 0.0, 255 is +1.0.
 *            The pages name only the signed code; this is its plainest
 *            unsigned form.
 *   QB_NF4   16 normal-quantile values in [-1, 1], two codes per byte.
 *   QB_FP4   E2M1 minifloat / 6, sign-magnitude nibble, two codes per byte.
 * 4-bit packing: element 2k is the high nibble of byte k, element 2k+1 the low
 * nibble; an odd count leaves the last low nibble 0.
 * Encoding: nearest entry of value/absmax, a tie going to the entry of smaller
 * magnitude; a block whose absmax is 0 gets the code of 0.0.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers unless marked "host".  The caller
 *     owns every buffer: libqb never allocates device memory and keeps no state
 *     between calls except its constant tables (and the one scratch array of
 *     qb_multi_tensor_step_noalloc).  Every entry point is safe to
 *     call from several host threads at once, with two exceptions whose
 *     calls on one device must not overlap in time (see their descriptions):
 *     qb_multi_tensor_step_noalloc, whose calls on one device share its
 *     scratch array, and qb_paged_optimizer_step, whose calls on one device
 *     share internal copy streams and events.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; no entry point synchronizes the device.
 *   - Arguments are validated before anything is enqueued; on any error
 *     nothing runs and nothing is written.  A failed launch returns QB_EHIP.
 *     No C++ exception crosses this interface.
 *   - Device pointers must be 16-byte aligned (QB_EALIGN otherwise).
 *   - n == 0 is a no-op returning QB_OK.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified codes.
 *   - blocksize is a power of two in [64, 4096]; the number of blocks must be
 *     below 2^31.
 */
#ifndef QB_H
#define QB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QB_OK = 0,
    QB_EINVAL = 1,        /* a null pointer, bad size, bad enum or bad hyperparameter */
    QB_EALIGN = 2,        /* a device pointer is not 16-byte aligned */
    QB_EUNSUPPORTED = 3,  /* a valid but unsupported combination */
    QB_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
    QB_EWORKSPACE = 5,    /* the workspace is too small */
    QB_EINIT = 6          /* the constant tables could not be built or uploaded */
} qb_status;

typedef enum { QB_F32 = 0, QB_F16 = 1, QB_BF16 = 2 } qb_dtype;

typedef enum { QB_DYN8 = 0, QB_NF4 = 1, QB_FP4 = 2, QB_UDYN8 = 3 } qb_code;

/*
 * Nested ("double") quantization state of the per-block absmax (page
 * "Bitsandbytes" (Transformers docs), section İç içe nicelleştirme: a second
 * quantization of the constants of the first, about 0.4 bit per parameter).
 * The nb = ceil(n / blocksize) fp32 absmax values a_j are centred on their mean
 *   offset = the exact mean of a_j, rounded once to fp32,
 * and d_j = a_j - offset (fp32) is quantized with QB_DYN8 in blocks of
 * blocksize2.  The decoded constant is dyn8[codes_j] * absmax2[j / blocksize2]
 * + offset (two rounded fp32 operations).
 */
typedef struct {
    uint8_t* codes;      /* [nb] QB_DYN8 codes of a_j - offset */
    float*   absmax2;    /* [ceil(nb / blocksize2)] */
    float*   offset;     /* [1] */
    int32_t  blocksize2; /* power of two in [64, 4096]; 256 is the usual value */
    void*    ws;         /* workspace of qb_dq_workspace_bytes(n, blocksize) bytes; used by qb_quantize only */
    size_t   ws_bytes;
} qb_dq;

/*
 * Hyperparameters of one AdamW step (pages: "bitsandbytes - Quantização de
 * LLM", section Workflow 3, where the 8-bit optimizer replaces AdamW with the
 * same lr, betas and eps; "Py之bitsandbytes", section 使用8位优化器).  They are
 * real numbers: every per-element scalar (beta1, 1-beta1, beta2, 1-beta2,
 * lr/(1-beta1^t), 1/sqrt(1-beta2^t), 1-lr*weight_decay, eps) is computed in
 * binary64 and rounded once to binary32.  step is the 1-based step t.
 * Requirements: 0 <= beta1, beta2 < 1; eps > 0; lr, weight_decay finite, >= 0;
 * step >= 1.
 */
typedef struct {
    double  lr;
    double  beta1;
    double  beta2;
    double  eps;
    double  weight_decay;
    int32_t step;
} qb_adamw_hparams;

/*
 * The fused 8-bit optimizers.  The pages list 8-bit Adam, AdamW, SGD, RMSprop
 * and Lion as drop-in replacements that keep their optimizer's
 * hyperparameters (page "bitsandbytes深度解析", section 优化器模块深度分析; page
 * "Py之bitsandbytes", sections 1 and 使用8位优化器).  Each follows its usual
 * definition, every state tensor held as block-wise QB_DYN8 codes with one fp32
 * absmax per block (state 1; state 2 for the two-state kinds):
 *   QB_ADAMW    state 1 = m, state 2 = v; decoupled weight decay (as
 *               qb_adamw8bit_step).
 *   QB_ADAM     state 1 = m, state 2 = v; L2 decay: g <- g + wd*p, then the
 *               bias-corrected Adam update.
 *   QB_LION     state 1 = m:  c = b1*m + (1-b1)*g;  p <- p*(1-lr*wd) - lr*sign(c);
 *               m <- b2*m + (1-b2)*g.
 *   QB_SGD      state 1 = momentum buffer (beta1 = momentum, in (0, 1)):
 *               g <- g + wd*p; buf <- g at step 1, else momentum*buf +
 *               (1-dampening)*g; p <- p - lr*(nesterov ? g + momentum*buf : buf).
 *   QB_RMSPROP  state 1 = v (beta2 = alpha):  g <- g + wd*p;
 *               v <- alpha*v + (1-alpha)*g*g;  p <- p - lr*g/(sqrt(v) + eps).
 * The layer-wise kinds (8-bit LARS and LAMB are listed beside them on page
 * "Py之bitsandbytes", section 1; the pages give no formulas, so these follow
 * the published definitions) scale each tensor's step by a ratio of norms over
 * that whole tensor, one tensor being one layer:
 *   QB_LAMB     state 1 = m, state 2 = v (You et al., 2019):  Adam's moments,
 *               r = (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps),  u = r + wd*p,
 *               p <- p - lr*ratio*u  with ratio = |p| / |u|.
 *   QB_LARS     state 1 = momentum buffer (beta1 = momentum, in [0, 1);
 *               You, Gitman and Ginsburg, 2017):
 *               ratio = trust_coefficient*|p| / (|g| + wd*|p|),
 *               buf <- momentum*buf + lr*ratio*(g + wd*p),  p <- p - buf.
 *   The norms (of p, and of u or g) and the ratio are binary64, a zero norm
 *   makes the ratio 1, and the step takes S = (float)(lr*ratio) as one
 *   binary32 scalar.  They need a workspace for the norms: only
 *   qb_multi_tensor_optimizer_step runs them (one tensor is a call with
 *   count 1).
 * The never-negative state (v of QB_ADAMW, QB_ADAM and QB_LAMB; the state of
 * QB_RMSPROP) may be held in QB_UDYN8 instead (hp->v_code): the same bytes,
 * with twice the resolution in every decade, which halves its worst
 * quantization error relative to the block absmax (0.0035 against 0.0070).
 * Its fresh state is code 0 (0.0).  A state written with one code must be
 * stepped with the same code.
 * The states and their codes are bit-exact against an IEEE binary32 evaluation
 * of these formulas (each operation rounded on its own, IEEE square root and
 * division).  So is p' for every kind but AdamW and LAMB, whose states never
 * read p: there p' takes hardware square root and reciprocal and is within
 * 1e-6 relative.  The layer-wise kinds add their norms in a fixed order of
 * their own (run to run the same bits); an evaluation that adds in another
 * order can differ in the last bits of the binary64 sums, which changes S only
 * when the ratio lies that close to a binary32 rounding boundary.
 */
typedef enum { QB_ADAMW = 0, QB_ADAM = 1, QB_LION = 2, QB_SGD = 3, QB_RMSPROP = 4, QB_LAMB = 5, QB_LARS = 6 } qb_optimizer;

/* Hyperparameters of one step of any kind (unused fields are ignored). */
typedef struct {
    qb_optimizer kind;
    double  lr;
    double  beta1;         /* Adam(W), Lion: beta1; SGD: momentum */
    double  beta2;         /* Adam(W), Lion: beta2; RMSprop: alpha */
    double  eps;           /* Adam(W), RMSprop */
    double  weight_decay;
    double  dampening;     /* SGD */
    int32_t nesterov;      /* SGD: 0 or 1 (1 needs dampening 0) */
    int32_t step;          /* t >= 1 */
    double  trust_coefficient;   /* LARS: eta > 0 */
    qb_code v_code;        /* code of the never-negative state: QB_DYN8 (0, the
                              default) or QB_UDYN8 (QB_ADAMW, QB_ADAM, QB_LAMB,
                              QB_RMSPROP only) */
} qb_optim_hparams;

/* One tensor of a multi-tensor step; the fields are those of qb_adamw8bit_step
 * (m, absmax_m: state 1; v, absmax_v: state 2, ignored by one-state kinds).
 * p holds n values of the call's parameter dtype (fp32 for qb_multi_tensor_step). */
typedef struct {
    void*       p;
    const void* g;
    uint8_t*    m;
    uint8_t*    v;
    float*      absmax_m;
    float*      absmax_v;
    int64_t     n;
} qb_tensor;

/*
 * One tensor of a grouped quantization; the fields are those of qb_quantize.
 * A plain tensor gives absmax and leaves c2, absmax2, offset NULL; a nested
 * one gives c2, absmax2, offset (the outputs of qb_dq) and absmax NULL.
 */
typedef struct {
    const void* x;
    uint8_t*    codes;
    float*      absmax;
    uint8_t*    c2;
    float*      absmax2;
    float*      offset;
    int64_t     n;
} qb_quant_tensor;

/*
 * One tensor of a grouped dequantization; the fields are those of
 * qb_dequantize.  A plain tensor gives absmax and leaves c2, absmax2, offset
 * NULL; a nested one gives c2, absmax2, offset (the qb_dq fields) and absmax
 * NULL.
 */
typedef struct {
    const uint8_t* codes;
    const float*   absmax;
    const uint8_t* c2;
    const float*   absmax2;
    const float*   offset;
    void*          y;
    int64_t        n;
} qb_dequant_tensor;

/*
 * qb_quantize -- block-wise quantization (pages cited at the top; NF4: page
 * "Bitsandbytes", section Normal Float 4 (NF4); FP4: page "Quantize 🤗
 * Transformers models", section FP4 quantization).
 *   x       [n] input of dtype xdt (fp32, fp16 or bf16).
 *   code    QB_DYN8 (codes: n bytes) or QB_NF4 / QB_FP4 (codes: ceil(n/2) bytes);
 *           QB_UDYN8 serves only the optimizer states (QB_EINVAL here).
 *   absmax  [ceil(n/blocksize)] fp32 block absmax out; must be NULL when dq is given.
 *   dq      NULL, or the nested state to fill (codes, absmax2, offset; the
 *           workspace holds the fp32 absmax while the call runs).
 * Outputs are fully overwritten.  One kernel, or four with dq (clear the
 * workspace's exponent bins, quantize, exact mean of the absmax, quantize
 * absmax - mean), all on `stream`.
 */
qb_status qb_quantize(const void* x, qb_dtype xdt, int64_t n, qb_code code, int32_t blocksize,
                      uint8_t* codes, float* absmax, const qb_dq* dq, void* stream);

/*
 * qb_normalize -- the normalized values of block-wise quantization, the step
 * between the block absmax and the encoding (each block is scaled by its own
 * absmax: "8-bit Optimizers via Block-wise Quantization" abstract, quoted on
 * page "Py之bitsandbytes", section 2), computed by the quantize kernels' own
 * quotient: out[i] = RN(x[i] / absmax[i / blocksize]) in binary32, equal to
 * IEEE division bit for bit (a zero x keeps its sign), and +0 where that
 * absmax is 0.  For inspection, e.g. counting values that lie within an ulp
 * of a code midpoint.
 *   x          [n] of dtype xdt.
 *   absmax     [ceil(n/blocksize)] fp32, finite, >= 0, with |x[i]| <=
 *              absmax[i / blocksize] (as qb_quantize writes it); other values
 *              give unspecified results.
 *   blocksize  any value >= 1 (1: one absmax per element).
 *   out        [n] fp32, fully overwritten.
 * One kernel.  QB_EINVAL for n < 0, blocksize < 1 or a NULL pointer with n > 0.
 */
qb_status qb_normalize(const void* x, qb_dtype xdt, int64_t n, const float* absmax, int32_t blocksize, float* out,
                       void* stream);

/*
 * qb_multi_tensor_quantize -- qb_quantize on `count` tensors (same input
 * dtype, code, block size and nested block size for all) in one kernel launch,
 * or four with nesting; the result equals a loop of single-tensor calls, bit
 * for bit.  Quantizing all weights of a model at load time (page
 * "Bitsandbytes", sections Normal Float 4 (NF4) and İç içe nicelleştirme) this
 * way avoids one launch ramp per tensor.
 *   tensors     host array of `count` descriptors (read during the call only);
 *               either every tensor is nested or none (else QB_EUNSUPPORTED).
 *   blocksize2  block size of the nested level (ignored without nesting).
 *   ws          device workspace of
 *               qb_multi_tensor_quantize_workspace_bytes(tensors, count,
 *               blocksize) bytes: tables of the tensors, copied in on
 *               `stream`, and with nesting the exponent bins and the fp32
 *               absmax of every tensor (4 bytes per block) while the call runs.
 * Tensors with n == 0 are skipped.  count == 0 is a no-op.
 */
qb_status qb_multi_tensor_quantize(const qb_quant_tensor* tensors, int32_t count, qb_dtype xdt, qb_code code,
                                   int32_t blocksize, int32_t blocksize2, void* ws, size_t ws_bytes,
                                   void* stream);
size_t qb_multi_tensor_quantize_workspace_bytes(const qb_quant_tensor* tensors, int32_t count,
                                                int32_t blocksize);

/*
 * qb_dequantize -- y_i = ydt(table[c_i] * s_b), one fp32 multiply then a
 * round-to-nearest-even conversion (page "Bitsandbytes", section on
 * dequantizing a model; compute dtype: page "Quantize 🤗 Transformers models",
 * section Change the compute dtype).  s_b is absmax[b], or with dq the decoded
 * nested constant of block b (dq->ws is not used).
 *   codes  [n] (DYN8) or [ceil(n/2)] (NF4/FP4);  y [n] of dtype ydt.
 */
qb_status qb_dequantize(const uint8_t* codes, const float* absmax, const qb_dq* dq, qb_code code,
                        int32_t blocksize, int64_t n, void* y, qb_dtype ydt, void* stream);

/*
 * qb_dequant_matmul -- y = x W^T with the weights W held in 4 bits: the
 * product of a 4-bit layer in its compute dtype (page "Bitsandbytes",
 * section QLoRA: Hesaplama veri türü; page "Quantize 🤗 Transformers models",
 * sections Change the compute dtype and Using NF4).  Every weight is first
 * dequantized exactly as by qb_dequantize into the compute dtype xdt, then the
 * products are summed in binary32 (fused in one kernel: the dequantized matrix
 * is never written to memory).
 *   x       [M, K] row-major, dtype xdt (QB_F32, QB_F16 or QB_BF16), 16-byte aligned.
 *   codes   W [N, K] row-major (a layer's [out, in] weight), NF4 or FP4 codes,
 *           two per byte as qb_quantize writes them; 16-byte aligned.
 *   absmax  [ceil(N*K / blocksize)] fp32, or NULL with dq (nested constants:
 *           dq->codes, absmax2, offset, blocksize2; dq->ws is not used).
 *   y       [M, N] row-major, dtype xdt, 16-byte aligned; each output is the
 *           binary32 sum rounded once to xdt.
 * Requirements: K a positive multiple of 32 below 2^24; M, N >= 0 (either 0: no-op).
 * Performance: up to 64 rows of x one wave per 16 weight rows streams W once
 * (up to 8 16-bit rows of at most 64 KiB in all are staged in LDS first);
 * from 65 rows (xdt 16-bit, K a multiple of 128) an LDS-tiled kernel shares x
 * across 64- or 128-row tiles and dequantizes W once per tile.  With M in the
 * thousands, dequantizing once and calling a GEMM library is faster.
 * Accuracy: each product of two xdt values is exact in binary32; the K-term
 * sums are added in an order of the kernel's own (fixed: the same bits on
 * every run), so y is within (K+2) 2^-23 sum_k |x_mk w_nk| of the exact
 * product before its final rounding.
 */
qb_status qb_dequant_matmul(const void* x, qb_dtype xdt, int64_t M, int64_t K, const uint8_t* codes,
                            const float* absmax, const qb_dq* dq, qb_code code, int32_t blocksize, int64_t N,
                            void* y, void* stream);

/*
 * One weight of qb_dequant_matmul_grouped: codes, absmax / nested constants
 * and y as for qb_dequant_matmul; N its rows (the layer's output features).
 * A plain weight gives absmax and leaves c2, absmax2, offset NULL; a nested
 * one gives c2, absmax2, offset (the qb_dq fields) and absmax NULL.
 */
typedef struct {
    const uint8_t* codes;
    const float*   absmax;
    const uint8_t* c2;
    const float*   absmax2;
    const float*   offset;
    void*          y;
    int64_t        N;
} qb_matmul_weight;

#define QB_MATMUL_GROUP_MAX 8

/*
 * qb_dequant_matmul_grouped -- qb_dequant_matmul for up to QB_MATMUL_GROUP_MAX
 * weights that multiply the same activations (a layer's query, key and value
 * projections; its gate and up projections): y_i = x W_i^T, each y_i bit for
 * bit the y of a qb_dequant_matmul call on weight i.  Same page citations as
 * qb_dequant_matmul.
 *   x, xdt, M, K         as for qb_dequant_matmul (one x for all weights).
 *   weights              host array of `count` descriptors (read during the
 *                        call only); every weight is plain or every one is
 *                        nested (else QB_EUNSUPPORTED); code, blocksize and
 *                        blocksize2 (nested only) are shared.
 * Weights with N == 0 are skipped (their pointers are not looked at);
 * count == 0 or M == 0 is a no-op;
 * count > QB_MATMUL_GROUP_MAX is QB_EINVAL.  Up to 64 rows of x (and for
 * binary32 x, or K not a multiple of 128, at any M) the column tiles of all
 * weights are one kernel launch, so small-batch projections fill the GPU
 * together; in the LDS-tiled regime it launches once per weight.
 */
qb_status qb_dequant_matmul_grouped(const void* x, qb_dtype xdt, int64_t M, int64_t K,
                                    const qb_matmul_weight* weights, int32_t count, qb_code code,
                                    int32_t blocksize, int32_t blocksize2, void* stream);

/*
 * qb_multi_tensor_dequantize -- qb_dequantize on `count` tensors in ONE kernel
 * launch (same code, block size, nested block size and output dtype for all;
 * the result equals a loop of single-tensor calls, bit for bit).  Dequantizing
 * the weights of many layers at once (page "Bitsandbytes", section on
 * dequantizing a model) this way avoids one launch ramp per tensor.
 *   tensors     host array of `count` descriptors (read during the call only);
 *               either every tensor is nested or none (else QB_EUNSUPPORTED).
 *   blocksize2  block size of the nested level (ignored without nesting).
 *   ws          device workspace of qb_multi_tensor_workspace_bytes(count)
 *               bytes, filled with a table of the tensors on `stream` (so it
 *               must not be reused by another stream until the call has run).
 * Tensors with n == 0 are skipped.  count == 0 is a no-op.
 */
qb_status qb_multi_tensor_dequantize(const qb_dequant_tensor* tensors, int32_t count, qb_code code,
                                     int32_t blocksize, int32_t blocksize2, qb_dtype ydt, void* ws,
                                     size_t ws_bytes, void* stream);

/*
 * qb_adamw8bit_step -- one fused AdamW step with both moments held as block-wise
 * QB_DYN8 codes (abstract quoted on "Py之bitsandbytes", section 2: 8-bit
 * optimizer state with block-wise dynamic quantization; "bitsandbytes -
 * Quantização de LLM", section Workflow 3: 2 bytes of state per parameter).
 * Per block of `blocksize` elements, in one kernel:
 *   m = dyn8[m_i]*absmax_m[b], v = dyn8[v_i]*absmax_v[b]
 *   m' = b1*m + (1-b1)*g,  v' = b2*v + (1-b2)*g*g
 *   p' = p*(1-lr*wd) - lr/(1-b1^t) * m' / (sqrt(v')/sqrt(1-b2^t) + eps)
 *   absmax_m[b] = max|m'|, absmax_v[b] = max|v'|, m_i, v_i = codes of m', v'.
 *   p          [n] fp32, in place.     g [n] of dtype gdt, read only; must not alias p.
 *   m, v       [n] uint8 codes, in place.  Fresh state: every code 127 (0.0), absmax 0.
 *   absmax_*   [ceil(n/blocksize)] fp32, in place.
 * The state codes and absmax are bit-exact against an IEEE binary32 evaluation
 * of the formulas above; p' uses hardware square root and reciprocal and is
 * within 1e-6 relative of it.
 */
qb_status qb_adamw8bit_step(float* p, const void* g, qb_dtype gdt, int64_t n, uint8_t* m, uint8_t* v,
                            float* absmax_m, float* absmax_v, int32_t blocksize,
                            const qb_adamw_hparams* hp, void* stream);

/*
 * qb_multi_tensor_step -- qb_adamw8bit_step on `count` tensors in ONE kernel
 * launch (blocks never span tensors; the result equals a loop of single-tensor
 * calls, bit for bit).
 *   tensors   host array of `count` descriptors (read during the call only).
 *   ws        device workspace of qb_multi_tensor_workspace_bytes(count) bytes;
 *             the call copies a table of the tensors (pointers, sizes, first
 *             tile numbers, and a coarse index from tile ranges to tensors)
 *             into it on `stream`, so ws must not be reused by another stream
 *             until the step has run.
 * Tensors with n == 0 are skipped.  count == 0 is a no-op.
 */
qb_status qb_multi_tensor_step(const qb_tensor* tensors, int32_t count, qb_dtype gdt, int32_t blocksize,
                               const qb_adamw_hparams* hp, void* ws, size_t ws_bytes, void* stream);

/*
 * qb_multi_tensor_step_noalloc -- qb_multi_tensor_step without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * tensor table goes into the library's own scratch: a device array of 384 KiB
 * that every GPU the library runs on holds until the process ends.  No device
 * memory is allocated or freed (no hipMalloc, hipFree or allocating library
 * call); host-side staging reuses per-thread buffers of the library.
 *   count     at most 4096 (QB_EWORKSPACE beyond).
 * Other arguments, the result (bit for bit) and the errors are those of
 * qb_multi_tensor_step.  Every call on one GPU shares that GPU's scratch,
 * which keeps the last call's table: calls that overlap in time on one GPU
 * (other streams, other host threads) race and must not be made; calls on
 * one stream are ordered and safe.
 */
qb_status qb_multi_tensor_step_noalloc(const qb_tensor* tensors, int32_t count, qb_dtype gdt, int32_t blocksize,
                                       const qb_adamw_hparams* hp, void* stream);

/*
 * qb_optimizer8bit_step -- one fused 8-bit step of optimizer hp->kind (see
 * qb_optimizer above) on one tensor.  Arguments as qb_adamw8bit_step, with
 * state1/absmax1 in place of m/absmax_m and state2/absmax2 in place of
 * v/absmax_v; state2 and absmax2 are ignored (may be NULL) for the one-state
 * kinds.
 * Parameter dtype pdt: QB_F32 (any gdt), or QB_F16 / QB_BF16 with gdt equal
 * to it (16-bit training without binary32 master weights, e.g. fp16 mixed
 * precision next to the 8-bit optimizer: "bitsandbytes - Quantização de LLM",
 * section Workflow 3).  A 16-bit parameter is widened to binary32 (exactly),
 * updated by the same binary32 formulas and rounded once, to nearest even,
 * back to its dtype; other pairs give QB_EUNSUPPORTED.  Fresh state: every code of 0.0 (127; 0 for a state in
 * QB_UDYN8), absmax 0.  A v_code other than QB_DYN8 or QB_UDYN8, or QB_UDYN8 for a kind without a never-negative
 * state, gives QB_EINVAL.  Invalid
 * hyperparameters for the kind (ranges above; lr, weight_decay >= 0) give
 * QB_EINVAL before anything is launched; the layer-wise kinds give
 * QB_EUNSUPPORTED (they run through qb_multi_tensor_optimizer_step).
 * 32-bit fallback: with absmax1 == NULL (and absmax2 == NULL) the states stay
 * binary32: state1 / state2 are float[n] arrays updated in place by the same
 * formulas, with no quantization.  This is the pages' policy for small or
 * chosen tensors (page "Py之bitsandbytes", sections 如果需要高精度的参数 and
 * 更改单个参数的位数: tensors under min_8bit_size elements, or marked 32-bit,
 * keep 32-bit state).  The multi-tensor step takes the same per tensor, so one
 * launch can mix 8-bit and 32-bit tensors.
 */
qb_status qb_optimizer8bit_step(const qb_optim_hparams* hp, void* p, qb_dtype pdt, const void* g, qb_dtype gdt,
                                int64_t n, uint8_t* state1, uint8_t* state2, float* absmax1, float* absmax2,
                                int32_t blocksize, void* stream);

/*
 * qb_multi_tensor_optimizer_step -- qb_optimizer8bit_step on `count` tensors in
 * one kernel launch (one parameter dtype pdt and gradient dtype gdt for all);
 * tensors, ws as for qb_multi_tensor_step, except that ws
 * holds qb_optimizer_workspace_bytes(hp, tensors, count, blocksize) bytes.
 * The layer-wise kinds (QB_LAMB, QB_LARS) take three launches on `stream`:
 * partial sums of the squared norms per group of optimizer tiles, one
 * workgroup per tensor that adds them in a fixed order and forms S, then the
 * fused step; the partial sums and the S of every tensor live in ws.
 */
qb_status qb_multi_tensor_optimizer_step(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count,
                                         qb_dtype pdt, qb_dtype gdt, int32_t blocksize, void* ws, size_t ws_bytes,
                                         void* stream);

/*
 * qb_paged_optimizer_step -- the multi-tensor 8-bit step with the optimizer
 * states held in host memory: the paged 8-bit optimizer of page
 * "bitsandbytes - Quantização de LLM", section Workflow 3 (optimizer
 * "paged_adamw_8bit"), for models whose states do not fit beside the weights.
 * Each tensor is cut into pages of page_params parameters; per page the
 * state codes and absmax are copied to a device staging slot, the fused step
 * runs on the page, and the states are copied back.  Two staging slots and
 * two internal copy streams (host to device, device to host; default priority)
 * overlap the copies of neighbouring pages with the step of the current one.
 * The result equals qb_multi_tensor_optimizer_step on device-resident states,
 * bit for bit (the same kernel per block).
 *   tensors      as for qb_multi_tensor_optimizer_step, with p and g in device
 *                memory and m, v, absmax_m, absmax_v in pinned host memory
 *                (hipHostMalloc, or torch's pin_memory); 8-bit states only.
 *   page_params  parameters per page: a positive multiple of blocksize.
 *   ws           device staging of qb_paged_workspace_bytes(page_params,
 *                blocksize) bytes, 16-byte aligned.
 * Kinds: every element-wise kind (QB_ADAMW .. QB_RMSPROP); the layer-wise ones
 * give QB_EUNSUPPORTED (their norms need a whole tensor before any page moves).
 * Ordering: the call's work starts after the work already on `stream` and
 * `stream` waits for the last copy back, so later work on `stream` sees the
 * updated parameters and states.  Calls on one device share the internal
 * streams and events, so they must not be made from several host threads at
 * once; the states of a call must not be touched by the host until `stream`
 * has passed the call, and consecutive calls on the same states should use
 * the same `stream`.
 */
qb_status qb_paged_optimizer_step(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count, qb_dtype pdt,
                                  qb_dtype gdt, int32_t blocksize, int64_t page_params, void* ws, size_t ws_bytes,
                                  void* stream);

/* Device staging bytes of qb_paged_optimizer_step: two slots, each with two
 * code pages of page_params bytes and two absmax pages, 256-byte aligned.
 * 0 if page_params is not a positive multiple of a valid blocksize. */
size_t qb_paged_workspace_bytes(int64_t page_params, int32_t blocksize);

/*
 * User codes.  The pages list three 8-bit quantization types, quantile,
 * linear and dynamic, and a fast quantile estimation (page "Py之bitsandbytes",
 * section 1).  Besides the built-in dynamic code, a block-wise 8-bit
 * quantization can use any 256-entry code held in a device table of
 * qb_code_table_bytes() bytes (16-byte aligned): the entries (256 floats at
 * the start), their exact decision thresholds (nearest entry; the midpoint of
 * two entries is taken in binary64; a tie goes to the entry of smaller
 * magnitude, between equal magnitudes to the upper one), and an index of the
 * thresholds by 2^-11-wide bucket of the normalized value, so the encoder
 * searches only its value's bucket.  Write tables only through the two calls
 * below.
 *   qb_linear_code      host: the linear code k/127, k = -128..127 (returns 256).
 *   qb_prepare_code     host values[256] (finite, non-decreasing; else
 *                       QB_EINVAL) -> device table, copied on `stream`.
 *   qb_estimate_quantiles
 *                       device: the quantile code of x[n] straight into a
 *                       device table.  The quantiles at j/257 (j = 0..256) are
 *                       estimated over chunks of 4096 consecutive values, each
 *                       sorted on its own (the chunk's order statistic at
 *                       floor(j L / 257), L its length; -0 counts as +0): A_j is
 *                       the exact mean of the chunks' statistics, rounded once
 *                       to nearest-even binary64.  Entries = binary32 of
 *                       q_i / max|q| with q_i = (A_i + A_{i+1}) / 2 (binary64).
 *                       Deterministic, and independent of the order of the
 *                       chunks' additions.  averages: NULL, or device double[257]
 *                       (16-byte aligned) that receives A.  ws:
 *                       qb_quantile_workspace_bytes(n) bytes.  Three kernels.
 *   qb_quantize_code / qb_dequantize_code
 *                       as qb_quantize / qb_dequantize with 8-bit codes (codes:
 *                       n bytes) and no nesting, the code given by `table`.
 */
size_t    qb_code_table_bytes(void);
int32_t   qb_linear_code(float* out);
qb_status qb_prepare_code(const float* values, void* table, void* stream);
size_t    qb_quantile_workspace_bytes(int64_t n);
qb_status qb_estimate_quantiles(const void* x, qb_dtype xdt, int64_t n, void* table, double* averages, void* ws,
                                size_t ws_bytes, void* stream);
qb_status qb_quantize_code(const void* x, qb_dtype xdt, int64_t n, const void* table, int32_t blocksize,
                           uint8_t* codes, float* absmax, void* stream);
qb_status qb_dequantize_code(const uint8_t* codes, const float* absmax, const void* table, int32_t blocksize,
                             int64_t n, void* y, qb_dtype ydt, void* stream);

/* Workspace sizes (bytes) for qb_quantize with nesting, and for
 * qb_multi_tensor_step, qb_multi_tensor_optimizer_step and qb_multi_tensor_dequantize. */
size_t qb_dq_workspace_bytes(int64_t n, int32_t blocksize);
size_t qb_multi_tensor_workspace_bytes(int32_t count);

/* Workspace bytes of qb_multi_tensor_optimizer_step: qb_multi_tensor_workspace_bytes(count)
 * for the element-wise kinds; for the layer-wise kinds two tables of the
 * tensors (by optimizer tile and by norm group), 16 bytes per norm group (32
 * optimizer tiles of max(blocksize, 1024) elements of one tensor) and 4 bytes
 * per tensor.  0 when hp, tensors or a size is invalid. */
size_t qb_optimizer_workspace_bytes(const qb_optim_hparams* hp, const qb_tensor* tensors, int32_t count,
                                    int32_t blocksize);

/*
 * qb_codebook -- host: copy the decode table of `code` (indexed by stored code)
 * into out (256 floats for DYN8 and UDYN8, 16 for NF4/FP4).  Returns the entry
 * count, or -1 for a bad code or a failed table build.
 */
int32_t qb_codebook(qb_code code, float* out);

/*
 * qb_encoder_table -- host: the encoder's bucket table, for inspection and
 * tests.  Each entry is two uint32 words {threshold bits, payload}:
 *   DYN8: 2 x 1409 entries, those of n >= 0 and then those of n < 0; bucket
 *         b = (clamp(bits(|n|), 2^-22, 1.0) >> 17) - (bits(2^-22) >> 17), plus
 *         1409 for n < 0; the code is payload + (n >= threshold).
 *   UDYN8: 2817 entries, n >= 0; bucket b = (clamp(bits(n), 2^-22, 1.0) >> 16)
 *         - (bits(2^-22) >> 16); the code is payload + (n >= threshold).
 *   NF4/FP4: bucket b = n*16 + 16 rounded once to the nearest integer, ties
 *         to even (0..32); NF4: the code is payload + (n >= threshold); FP4:
 *         byte 0 of payload if n < threshold, else byte 1.
 * Copies at most `capacity` entries (2*capacity words) into out and returns the
 * table's entry count, or -1 on error.
 */
int32_t qb_encoder_table(qb_code code, uint32_t* out, int32_t capacity);

/* Static text for a status code. */
const char* qb_status_string(qb_status s);

#ifdef __cplusplus
}
#endif

#endif /* QB_H */
