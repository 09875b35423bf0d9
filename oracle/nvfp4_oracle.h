/*
 * nvfp4_oracle.h -- plain, slow CPU oracle for the NVFP4 quantize / RHT / dequantize / GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or calls this code;
 * only the test suite, the package smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no source with the HIP kernels.
 *
 * What it follows:
 *  - NVFP4 = 4-bit E2M1 elements in 16-element blocks, one E4M3 scale per block and one FP32
 *    scale per tensor ("NVIDIA Introduces a 4-Bit Pretraining Methodology Using NVFP4 ...",
 *    aissential.tech, Summary).  The two-level micro-scaling encoding, 2D block quantization,
 *    the random Hadamard transform and stochastic rounding for gradients are named in the
 *    hyper.ai (fr) story on NVFP4 pretraining in JAX/MaxText; the 16x16 RHT on Wgrad inputs and
 *    2D 16x16 weight scaling in the same aissential.tech article, Method.
 *  - Four-over-Six: per block, choose between two grid targets for the block maximum
 *    (hyper.ai (de) story on the Nemotron 3 Ultra NVFP4 checkpoint).
 *  The pages print no formula; every arithmetic step below is the plain reading fixed in the
 *  accompanying design notes (tensor scale = amax/(6*448), block scale = block amax/6 clamped to
 *  the E4M3 maximum 448, E2M1 grid {0,0.5,1,1.5,2,3,4,6} with round-to-nearest-even).
 *
 * Precision: quantize decisions are taken in IEEE binary32 exactly as listed (each written
 * operation is one correctly rounded fp32 operation, fma only where written); the GEMM reference
 * and its error bound are accumulated in binary64.
 *
 * Parity pins: every function here is pinned by the CPU test suite against closed forms, library
 * routines (PyTorch's float8_e4m3fn cast and Philox4_32 engine), hand-computed worked examples,
 * invariants and brute force.  Throughput figures are measured only (parity unpinned).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Mode bits.  Same meaning as the library's public flags (an interface both sides must agree on). */
#define OR_COLWISE       1u  /* logical Y = x^T: blocks run along x's dim 0            */
#define OR_BLOCK2D       2u  /* one scale per 16x16 tile of Y                            */
#define OR_SR            4u  /* stochastic rounding of elements (Philox4x32-10)          */
#define OR_FOUR_OVER_SIX 8u  /* per block (1D) or 16x16 tile (2D), target 6 or 4 by lower SSE */
#define OR_TS_FOR_FOUR  16u  /* tensor scale amax / (4*448): a block scale for target 4 never clamps */
#define OR_SCALE_SEARCH 32u  /* per 1D block, target in {6, 5.5, 5, 4.5, 4} by lowest block SSE */

#define OR_DT_F32  0
#define OR_DT_BF16 1

/* ---- format primitives ------------------------------------------------------------------- */
float    or_e2m1_value(int code);          /* code 0..15: sign<<3 | magnitude index               */
int      or_e2m1_rne_index(float v);       /* v >= 0: index 0..7 of the nearest grid value, ties
                                              to the even index, saturating at 6                 */
float    or_e4m3_value(int byte);          /* E4M3FN decode (NaN for 0x7F / 0xFF)                 */
int      or_e4m3_rne(float s);             /* s in [0,448]: nearest E4M3FN byte, ties to even     */
void     or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t or_rht_sign_word(uint64_t sign_seed);     /* low 16 bits used                            */
void     or_rht16(float u[16], uint32_t sign_word); /* in place: (1/4) H16 D u, fixed butterfly    */

/* vectorised helpers for the tests */
void or_e2m1_rne_array(const float *v, int64_t n, uint8_t *idx);
void or_e4m3_rne_array(const float *s, int64_t n, uint8_t *bytes);
void or_philox_array(const uint32_t *ctr4, const uint32_t *key2, int64_t n, uint32_t *out4);
void or_rht16_array(float *u, int64_t nchunks, uint32_t sign_word); /* or_rht16 on each 16-chunk */

/* ---- quantize ----------------------------------------------------------------------------
 * x: rows x cols, row-major with leading dimension ldx (elements), dtype OR_DT_F32 or OR_DT_BF16
 * (bf16 given as raw uint16 bits, widened exactly).  Logical Y[R x K]: ROW mode R=rows, K=cols;
 * COLWISE R=cols, K=rows.  Outputs (caller-allocated host buffers):
 *   data   [R][K/2]   packed codes, low nibble = even k
 *   scales [R][K/16]  (1D) or [R/16][K/16] (BLOCK2D), E4M3 bytes
 *   ts     1 float    tensor scale = amax / 2688 (amax / 1792 with OR_TS_FOR_FOUR)
 *   rht_out (nullable, only with use_rht) [R][K] fp32 transformed Y
 *   sse2   (nullable) [0] = sum of chosen block SSE, [1] = sum of plain (target 6) block SSE;
 *          filled for FOUR_OVER_SIX and SCALE_SEARCH only
 * Block SSE: fp32, diff = RN(y - xhat), acc = fma(diff, diff, acc) in block order (1D).  For a
 * 16x16 tile every element contributes RN(diff * diff) and the 256 squares are summed over a
 * quad tree: each 2n x 2n block is RN(RN(TL + BR) + RN(TR + BL)) of its four n x n blocks (TL:
 * top-left, BR: bottom-right, ...), down to single elements.  Transposition maps TL and BR onto
 * themselves and swaps TR with BL, so a tile and its transpose get the same sum and the same
 * choice: quantizing W^T equals transposing the quantized W.  A candidate replaces the current
 * choice only if its SSE is strictly lower (candidates in the order listed above).
 * Returns 0 on success, nonzero on an unsupported shape / mode.                                */
int or_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                uint64_t seed, uint32_t stream_id, int use_rht, uint64_t sign_seed,
                uint8_t *data, uint8_t *scales, float *ts, float *rht_out, double *sse2,
                int nthreads);

/* Row-wise 1D nearest-even quantization of an fp32 matrix y [rows][ldy] with a GIVEN tensor scale
 * ts (instead of amax / 2688): the same per-block steps as or_quantize with flags 0 (block scale
 * RN(RN(a_b / 6) / ts) clamped to 448 then E4M3 nearest-even; e = RN(1 / RN(S * ts)); codes the
 * nearest E2M1 value of |y| * e, ties to even, saturating at 6; ts == 0 gives zero scales and
 * signed-zero codes).  This is what a GEMM epilogue that quantizes its output under delayed
 * scaling computes (the tensor scale comes from an earlier maximum; this library's reading).
 * data [rows][cols/2], scales [rows][cols/16].  Returns 0, or 2 if cols % 16 != 0.            */
int or_quantize_given_ts(const float *y, int64_t rows, int64_t cols, int64_t ldy, float ts, uint8_t *data,
                         uint8_t *scales, int nthreads);

/* Four-over-Six tile error of one 16x16 tile (row-major, leading dimension ld) for grid target T
 * (6 or 4) under tensor scale ts: the block scale of the tile maximum for T (as or_quantize), the
 * nearest-even codes under it, and the quad-tree sum of the squared errors described above.
 * *sb_out (nullable) receives the scale byte.  For tests that build near-tie tiles.            */
float or_tile_sse_2d(const float *tile, int64_t ld, float ts, float T, uint8_t *sb_out);

/* Dequantize to fp32: y[r*K + k] = RN(RN(e2m1 * S) * ts). */
int or_dequantize(const uint8_t *data, const uint8_t *scales, float ts, int64_t R, int64_t K,
                  uint32_t flags, float *y);

/* ---- GEMM reference ------------------------------------------------------------------------
 * C[i][j] = ts_a*ts_b * sum_blocks S_a S_b sum_{k in block} q_a q_b, in binary64, for A [M x K]
 * and B [N x K] (both K-major NVFP4, each 1D or BLOCK2D per its flags).  bound[i][j] =
 * sum_k |a_ik| |b_jk| of the exactly dequantized operands.  Only the n_tiles rectangles
 * (row0, col0, h, w) given in tiles[4*t..] are computed; out is [M x N] row-major (ldc = N) and
 * untouched elsewhere.                                                                         */
int or_gemm_ref(const uint8_t *a_data, const uint8_t *a_scales, float a_ts, uint32_t a_flags,
                const uint8_t *b_data, const uint8_t *b_scales, float b_ts, uint32_t b_flags,
                int64_t M, int64_t N, int64_t K, const int64_t *tiles, int64_t n_tiles,
                double *c, double *bound, int nthreads);

/* W4A16 reference: C[i][j] = ts_b * sum_k a[i][k] * (q_b S_b)[j][k] in binary64, A given as bf16
 * bits [M][lda] (widened exactly), B an NVFP4 [N x K] operand (1D or BLOCK2D).  bound as above.
 * Tiles as for or_gemm_ref. */
int or_gemm_w4a16_ref(const uint16_t *a_bf16, int64_t lda, const uint8_t *b_data, const uint8_t *b_scales,
                      float b_ts, uint32_t b_flags, int64_t M, int64_t N, int64_t K, const int64_t *tiles,
                      int64_t n_tiles, double *c, double *bound, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
