/*
 * qb_stream.h -- HBM reference streams of the benchmark (libqb_stream.so).
 *
 * Not part of the block-wise quantization library: three plain streaming
 * kernels that bound what a kernel of libqb can reach on the same device and
 * in the same process, in the fastest plain form measured on MI355X (one
 * 16-byte non-temporal access per thread, one 256-thread workgroup per 1024
 * floats, each XCD on its own contiguous eighth of the buffer).  The
 * benchmark reports them beside the roofline figures.
 *
 * All pointers are DEVICE pointers, 16-byte aligned, owned by the caller;
 * n (floats) must be a positive multiple of 1024.  Work is enqueued on
 * `stream` (a hipStream_t, NULL = default stream).  Each call returns 0, or a
 * hipError_t code (invalid arguments: nothing is enqueued).
 *   qbs_copy    dst[i] = src[i]: n floats read, n written.
 *   qbs_read    reads src[0..n); writes sink[0..255] only if a thread's sum
 *               of its 4 values equals `never` exactly (pass a value
 *               the data cannot sum to, e.g. NaN, so nothing is written).
 *   qbs_write   dst[i] = value: n floats written.
 *
 * Access-pattern streams: the memory accesses of libqb's multi-tensor 8-bit
 * AdamW step and of its grouped nested 4-bit dequantize, on the caller's own
 * buffers, with no arithmetic (the same tiles, widths, non-temporal flags and
 * XCD-contiguous tile order).  `tensors` is a device array of `count`
 * descriptors, `tile_begin` a device array of count + 1 first tiles (the last
 * is the total, ntiles).
 *   qbs_adamw_pattern     descriptors {float* p; const uint16_t* g (bf16);
 *                         uint8_t* m, *v; float* absmax_m, *absmax_v;
 *                         int64_t n; int64_t pad} (64 bytes); block 2048,
 *                         one tile per block.  Every byte is written back
 *                         unchanged, so the step's state survives.
 *   qbs_dequant4_pattern  descriptors {const uint8_t* codes (4-bit, two per
 *                         byte), *c2; const float* absmax2, *offset;
 *                         uint16_t* y (bf16 out); int64_t n; int64_t pad[2]}
 *                         (64 bytes); block 64, second level 256, 8192
 *                         weights per tile.  y receives arbitrary values.
 */
#ifndef QB_STREAM_H
#define QB_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int qbs_copy(const float* src, float* dst, int64_t n, void* stream);
int qbs_read(const float* src, int64_t n, float never, float* sink, void* stream);
int qbs_write(float* dst, int64_t n, float value, void* stream);
int qbs_adamw_pattern(const void* tensors, const int64_t* tile_begin, int count, int64_t ntiles, void* stream);
int qbs_dequant4_pattern(const void* tensors, const int64_t* tile_begin, int count, int64_t ntiles, void* stream);

#ifdef __cplusplus
}
#endif

#endif
