/*
 * wgemm.h -- C ABI of the weight-quantised decode GEMM in libkvfp8.so (MI355X,
 * gfx950): bf16 activations times weights stored as INT4 (W4A16) or FP8 e4m3
 * (W8A16) codes.
 *
 * What it computes comes from the pages' weight compression: the Cloudflare
 * post "Smaller, faster, safer: running Kimi and GLM at scale", section
 * "Compressed model weights" (压缩模型权重), and the agentlenshq summary,
 * section "模型权重压缩以降低延迟": GLM's weights go from FP8 to INT4; decode
 * streams every weight once per token and is bound by memory bandwidth, so
 * it speeds up; the INT4 weights are expanded to a wider type before the
 * multiply (which is why prefill, compute-bound, slows down).  The pages
 * give neither the grouping nor the scale format; the readings below are
 * this library's.
 *
 * Quantisation (one bf16 scale per group of 128 consecutive input channels
 * of an output channel; weights must be finite):
 *   INT4: s = bf16(fl32(max|w| / 7)), q = clamp(rint(fl32(w * fl32(1/s))),
 *         -8, 7), ties to even; weight used = s * q.
 *   FP8:  s = bf16(fl32(max|w| / 448)), code = e4m3 of fl32(w * fl32(1/s))
 *         (OCP E4M3, RNE, saturating: the KV cache's encoder); weight used =
 *         s * dec(code).
 *   A group whose scale is 0 (all zero) gets codes 0.
 * GEMM: y[m][n] = sum_k x[m][k] * weight[n][k], products exact, fp32
 * accumulation (per group, then scaled), bf16 (RNE) result.
 *
 * Storage layout (packed codes):
 *   tiles of 16 output channels x 128 input channels, tile (t, g) at index
 *   t * (K/128) + g; inside a tile, lane l = 16*qq + nn (qq 0..3, nn 0..15)
 *   owns output channel 16t + nn and input channels 128g + 32j + 8qq + e
 *   (j 0..3, e 0..7).
 *   INT4: 16 bytes per lane; little-endian dword j holds the codes of (j, e)
 *         as unsigned nibbles q + 8, e = 2*(s%4) + s/4 in bits 4s..4s+3.
 *   FP8:  32 bytes per lane; byte 8j + e holds the code of (j, e).
 *   scales: bf16 [N/16][K/128][16]; element (t, g, nn) is the scale of
 *   output channel 16t + nn in group g.
 *
 * Conventions as in kvfp8.h: device pointers, asynchronous on `stream`,
 * status KVFP8_OK or a negative KVFP8_ERR_* (an error enqueues nothing), no
 * allocation, x / packed / y 16-byte aligned, scales 2-byte aligned.
 * Shapes: N a multiple of 16, K a multiple of 256 (KVFP8_ERR_SHAPE
 * otherwise); the GEMM takes 1 <= M <= 64 rows.
 */
#ifndef WGEMM_H
#define WGEMM_H

#include <stddef.h>
#include <stdint.h>

#include "kvfp8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sizes of the packed codes and the scale array (0 for an unsupported shape). */
size_t w4_packed_bytes(int32_t n, int32_t k);
size_t w8_packed_bytes(int32_t n, int32_t k);
size_t wq_scales_count(int32_t n, int32_t k);

/* Quantise bf16 weights w [N][K] (row-major) into packed codes and scales,
 * as above.  One launch; the inputs are read once. */
int w4_quantize_bf16(const uint16_t* w, int32_t n, int32_t k, uint8_t* packed, uint16_t* scales,
                     hipStream_t stream);
int w8_quantize_bf16(const uint16_t* w, int32_t n, int32_t k, uint8_t* packed, uint16_t* scales,
                     hipStream_t stream);

/* y bf16 [M][N] = x bf16 [M][K] times the packed weights, transposed.
 * num_splits: 0 = chosen by the library, else at most K/256; the K range is
 * cut into that many slices (for M > 16 with more than 16 activation rows'
 * worth of LDS, at most 8192 input channels per slice: KVFP8_ERR_UNSUPPORTED
 * otherwise).  One launch either way: with several slices their fp32 partials
 * go to `workspace` (device, 16-byte aligned, at least
 * wgemm_workspace_bytes(M, N, K, splits) bytes; 0 and NULL allowed for one
 * split), and the last block of each column group to finish adds them in
 * split order.  The workspace opens with ceil(N/16) uint32 counters, one
 * per 128-byte line (padded to 256 bytes), that must be zero before the
 * first call that uses it (e.g.
 * allocate it zeroed once); every call leaves them zero, so one workspace
 * serves any sequence of calls on one stream.  Calls that overlap in time
 * must not share a workspace. */
int32_t wgemm_auto_splits(int32_t m, int32_t n, int32_t k);
size_t wgemm_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t num_splits);
int w4a16_gemm(const uint16_t* x, int32_t m, const uint8_t* w_packed, const uint16_t* scales, int32_t n,
               int32_t k, int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* y,
               hipStream_t stream);
int w8a16_gemm(const uint16_t* x, int32_t m, const uint8_t* w_packed, const uint16_t* scales, int32_t n,
               int32_t k, int32_t num_splits, void* workspace, size_t workspace_bytes, uint16_t* y,
               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WGEMM_H */
