/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 quantize / RHT-quantize / dequantize / block-scaled GEMM
 * on AMD Instinct MI355X (gfx950).
 *
 * Format (NVFP4, the two-level micro-scaling encoding): 4-bit E2M1 elements in blocks of 16
 * consecutive elements along the contraction axis, one E4M3 scale per block and one FP32 scale per
 * tensor ("NVIDIA Introduces a 4-Bit Pretraining Methodology Using NVFP4 ...", aissential.tech,
 * Summary; hyper.ai (fr) story on NVFP4 pretraining with JAX/MaxText/TransformerEngine).
 * Readings this library fixes where the pages are silent:
 *   - element value      q in {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit; code = sign<<3 | index
 *   - tensor scale       ts = RN(amax / 2688)              (2688 = 6 * 448)
 *   - block scale        byte = E4M3_RNE(min(RN(RN(block_amax / T) / ts), 448)), T = 6 (or 4, see
 *                        NVFP4_FOUR_OVER_SIX); byte 0 when ts == 0
 *   - element encode     v = RN(|y| * RN(1 / RN(S * ts))), rounded to the E2M1 grid (nearest, ties
 *                        to the even code, saturating at 6) or stochastically (NVFP4_SR); the sign
 *                        bit is always copied from y
 *   - decode             y_hat = RN(RN(q * S) * ts)
 *   - packing            byte [r][k/2] = code(k even) | code(k odd) << 4
 * These steps are bit-exact: the same input gives the same bytes on every call and device.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are caller-owned device memory (PyTorch tensors in the Python
 *     binding); the library allocates nothing and keeps no state between calls.
 *   - All work is enqueued on `hip_stream` (a hipStream_t; NULL = the default stream) and the call
 *     returns after enqueue, without synchronising.
 *   - Arguments are validated on the host before anything is enqueued.  On an error the call
 *     returns the status below and enqueues nothing.  Errors never throw across the ABI.
 *   - Matrices are row-major with a leading dimension in elements.
 *   - Inputs are finite (NaN / Inf are not detected).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL                                       */
  NVFP4_ERR_SHAPE = 2,       /* negative size, K % 16 != 0, rows % 16 != 0 for 2D blocks, a
                                leading dimension smaller than the row, or an output descriptor
                                whose rows / k / flags do not match the call                        */
  NVFP4_ERR_ALIGN = 3,       /* a pointer not 16-byte aligned, or a leading dimension not a
                                multiple of 16 bytes                                                */
  NVFP4_ERR_UNSUPPORTED = 4, /* a flag / dtype combination this library does not implement        */
  NVFP4_ERR_HIP = 5          /* a HIP launch failed                                                 */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

enum {
  /* Quantize x^T instead of x: blocks run along x's dim 0 (e.g. the token dimension of a weight
   * gradient's inputs) and the output is stored K-major for the transposed matrix. */
  NVFP4_COLWISE = 1u << 0,
  /* One scale per 16x16 tile of the logical matrix (2D 16x16 weight scaling: aissential.tech
   * article, Method; hyper.ai (fr) story, "quantification par blocs 2D"). */
  NVFP4_BLOCK2D = 1u << 1,
  /* Stochastic rounding of elements (gradients; the hyper.ai (fr) story names it for keeping
   * gradients unbiased).  Random bits: Philox4x32-10 keyed by (lo32(seed), hi32(seed)) at counter
   * (lo32(i>>3), hi32(i>>3), stream_id, 0) with i = r*K + k the element's index in the logical
   * output; element i uses 16 bits r16 = word[(i&7)>>1] >> (16*(i&1)); it rounds up iff
   * (float)r16 < f * 65536 where f is its fractional position between the two grid neighbours.
   * Block scales are always round-to-nearest. */
  NVFP4_SR = 1u << 2,
  /* Four-over-Six (hyper.ai (de) story on the Nemotron 3 Ultra NVFP4 checkpoint): per 1D block,
   * map the block maximum to 6 or to 4, whichever gives the lower block squared error (fp32,
   * fused multiply-add in block order; a tie keeps 6).  ts is unchanged.  With NVFP4_BLOCK2D the
   * choice is made per 16x16 tile: each element's squared error is rounded to fp32 and the 256
   * squares are summed over a quad tree, each 2n x 2n block as (top-left + bottom-right) +
   * (top-right + bottom-left) of its n x n blocks.  That sum does not change under transposition,
   * so quantizing W^T (NVFP4_COLWISE) equals transposing the quantized W (nvfp4_transpose). */
  NVFP4_FOUR_OVER_SIX = 1u << 3,
  /* Tensor scale amax / (4 * 448) instead of amax / (6 * 448): a block scale for target 4 then
   * never clamps at the E4M3 maximum (a variant of Four-over-Six; combinable with every mode). */
  NVFP4_TS_FOR_FOUR = 1u << 4,
  /* Scale search (an ablation of Four-over-Six): per 1D block, the lowest squared error among the
   * targets 6, 5.5, 5, 4.5, 4 (tried in that order; a later target must be strictly better).  Not
   * with NVFP4_SR, NVFP4_FOUR_OVER_SIX or NVFP4_BLOCK2D. */
  NVFP4_SCALE_SEARCH = 1u << 5
};

/* Non-owning view of one NVFP4 tensor: logical matrix [rows x k], k contiguous (the contraction
 * axis).  For a grouped GEMM operand B, data / scales / tensor_scale are group-contiguous arrays
 * (see nvfp4_gemm). */
typedef struct {
  uint8_t *data;        /* device, [rows][k/2] packed codes, low nibble = even k                  */
  uint8_t *scales;      /* device, E4M3 bytes: [rows][k/16] (1D) or [rows/16][k/16] (BLOCK2D)    */
  float *tensor_scale;  /* device, ts (one fp32; one per group for a grouped B)                  */
  int64_t rows;         /* logical rows                                                          */
  int64_t k;            /* logical columns (contraction axis), multiple of 16                    */
  uint32_t flags;       /* NVFP4_BLOCK2D if the scales are 16x16-tile scales; other bits ignored */
} nvfp4_tensor;

/* Bytes of device workspace nvfp4_quantize / nvfp4_rht_quantize need for this shape and flags
 * (the per-workgroup partial maxima of the amax pass).  The workspace is fully rewritten by every
 * call before it is read; it needs no initialisation.  Calls that may overlap must use distinct
 * workspaces. */
size_t nvfp4_workspace_size(int64_t rows, int64_t cols, uint32_t flags);

/* Quantize x [rows x cols] (dtype NVFP4_F32 or NVFP4_BF16, leading dimension ldx elements) to
 * NVFP4.  Two kernels run on the stream: the tensor amax pass, then the block-scale / encode /
 * pack pass (which also writes *out->tensor_scale).
 * flags: any of NVFP4_COLWISE, NVFP4_BLOCK2D, NVFP4_SR, NVFP4_FOUR_OVER_SIX, NVFP4_TS_FOR_FOUR,
 *   NVFP4_SCALE_SEARCH, except SR with FOUR_OVER_SIX, SCALE_SEARCH or BLOCK2D, and SCALE_SEARCH
 *   with FOUR_OVER_SIX or BLOCK2D (NVFP4_ERR_UNSUPPORTED).
 * Logical matrix: Y = x (R = rows, K = cols), or Y = x^T with NVFP4_COLWISE (R = cols, K = rows).
 *   K % 16 == 0; with NVFP4_BLOCK2D also R % 16 == 0; with NVFP4_COLWISE also cols % 8 == 0.
 * out: caller-filled descriptor with rows == R, k == K, (flags & NVFP4_BLOCK2D) equal to the
 *   call's, and device buffers of R*K/2, R*K/16 (or R*K/256) and 4 bytes.
 * seed, stream_id: the stochastic-rounding key and stream (ignored without NVFP4_SR).
 * workspace: device, nvfp4_workspace_size() bytes, 16-byte aligned.
 * x, out->data and workspace must be 16-byte aligned and ldx * sizeof(dtype) a multiple of 16. */
int nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                   uint32_t flags, uint64_t seed, uint32_t stream_id, nvfp4_tensor *out,
                   void *workspace, void *hip_stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation and result, with the
 * amax pass's workspace in a library-owned 16 KiB device array (one per GPU, held until the process
 * ends) instead of a caller buffer.  The call allocates nothing; on its first use on a device it
 * looks the array's address up (hipGetSymbolAddress) with that device current.  Every call on one
 * GPU shares the array, so calls that may overlap on one GPU (different streams) race: serialise
 * them or use nvfp4_quantize with distinct workspaces.  Arguments, layouts and errors as
 * nvfp4_quantize; a shape whose workspace would exceed the array gives NVFP4_ERR_SHAPE (none of the
 * shapes nvfp4_quantize accepts does). */
int nvfp4_quantize_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                           uint32_t flags, uint64_t seed, uint32_t stream_id, nvfp4_tensor *out,
                           void *hip_stream);

/* As nvfp4_quantize, after a 16x16 random Hadamard transform of every 16-element block along K
 * (Wgrad inputs: aissential.tech article, Method; hyper.ai (fr) story, "transformation de Hadamard
 * aleatoire").  Each block u becomes (1/4) H16 D u with H16 the Sylvester Hadamard matrix and D the
 * diagonal of signs given by the low 16 bits of word 0 of Philox4x32-10 keyed by sign_seed at
 * counter (0, 0, 0, 1) (bit t set: u[t] is negated).  The transform runs as the radix-2 butterfly
 * with strides 1, 2, 4, 8 in fp32, then a multiply by 0.25.  Both operands of a GEMM must use the
 * same sign_seed so that the transforms cancel in the product.
 * rht_out: nullable device fp32 [R][K]; if given, the transformed Y is also written (for tests).
 * BLOCK2D is not supported with the transform. */
int nvfp4_rht_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx,
                       uint32_t flags, uint64_t seed, uint32_t stream_id, uint64_t sign_seed,
                       float *rht_out, nvfp4_tensor *out, void *workspace, void *hip_stream);

/* Grouped quantize (MoE expert weights, each with its own tensor scale; the routed experts are the
 * NVFP4 part of the hyper.ai (de) story's Nemotron 3 Ultra checkpoint): `groups` equally shaped tensors
 * x_g = x + g * group_stride elements (g = 0 .. groups-1, each [rows x cols] with leading dimension
 * ldx), quantized in one pair of launches.  Group g is exactly nvfp4_quantize(x_g, x_dtype, rows,
 * cols, ldx, flags, seed, stream_id + g, out_g, ...), where out_g is group g of out: out->rows == R
 * and out->k == K per group as for nvfp4_quantize, and out->data / out->scales / out->tensor_scale
 * hold `groups` consecutive tensors (R*K/2 and R*K/16 or R*K/256 bytes, one float each), the layout
 * of a grouped nvfp4_gemm weight.  Flags and shape rules as nvfp4_quantize.
 * groups: 1 .. 65535 and group_stride >= 0 elements with (groups - 1) * group_stride <= 2^36 (else
 * NVFP4_ERR_SHAPE); group_stride * sizeof(dtype) a multiple of 16 (else NVFP4_ERR_ALIGN).  workspace: device, groups * nvfp4_workspace_size() bytes,
 * 16-byte aligned.  All buffers are device memory owned by the caller; out must not overlap x. */
int nvfp4_quantize_grouped(const void *x, int x_dtype, int64_t groups, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t group_stride, uint32_t flags, uint64_t seed, uint32_t stream_id,
                           nvfp4_tensor *out, void *workspace, void *hip_stream);

/* Decode an NVFP4 tensor to y [in->rows x in->k] (dtype NVFP4_F32 or NVFP4_BF16, leading
 * dimension ldy elements): y = RN(RN(q * S) * ts), rounded once more to bf16 (nearest-even) for a
 * bf16 output.  Decoding NVFP4 weights to 16 bits is what a W4A16 fallback needs (hyper.ai (de)
 * story: Hopper switches to W4A16). */
int nvfp4_dequantize(const nvfp4_tensor *in, void *y, int y_dtype, int64_t ldy, void *hip_stream);

/* Block-scaled NVFP4 x NVFP4 GEMM with FP32 accumulation (native W4A4: hyper.ai (de) story; the
 * feed-forward GEMMs are where the training time goes: hyper.ai (fr) story):
 *   C[i][j] = ts_a * ts_b * sum_k (q_a[i][k] * S_a(i,k)) * (q_b[j][k] * S_b(j,k)),
 * i.e. C = A * B^T with A [M x K] = a (M = a->rows) and B [N x K] = b (N = b->rows), both K-major.
 * Each element product q*S is exact in fp16, the K sum accumulates in fp32, and ts_a*ts_b is applied
 * once at the end.  c: device, [M x N] with leading dimension ldc, dtype NVFP4_F32 or NVFP4_BF16.
 * Either operand may use 1D or BLOCK2D scales.
 * Grouped form (MoE experts): num_groups > 1 and group_row_offsets a HOST array of num_groups + 1
 * nondecreasing row offsets into A (offsets[0] == 0, offsets[G] == M).  Rows offsets[g] ..
 * offsets[g+1]-1 of A and C use group g's weight: b->rows is N (per group), b->data / b->scales
 * hold G consecutive [N x K] tensors and b->tensor_scale holds G floats.
 * a->data and b->data must be 16-byte aligned, c aligned to its element size; K % 16 == 0;
 * ldc >= N. */
int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype, int64_t ldc,
               int32_t num_groups, const int64_t *group_row_offsets, void *hip_stream);

/* Transpose of an NVFP4 tensor with 16x16 block scales: out = in^T, i.e. out codes [k x rows]
 * (out->rows == in->k, out->k == in->rows), out scales the transposed [k/16][rows/16] grid, and the
 * same tensor scale.  With 2D scaling every 16x16 tile shares one scale, so this equals quantizing
 * Y^T directly (bit for bit): a weight quantized once for the forward GEMM feeds the backward-data
 * GEMM, whose contraction runs along the other dimension.  (The recipe scales weights in 2D 16x16
 * blocks: aissential.tech article, Method; hyper.ai (fr) story.  That one 2D quantization serves
 * both GEMMs is this library's reading: 16x16 tiles map onto 16x16 tiles under transposition.)
 * Both descriptors must carry NVFP4_BLOCK2D (else NVFP4_ERR_UNSUPPORTED); rows and k multiples of
 * 16; data 16-byte aligned; all buffers device memory owned by the caller; in and out must not
 * overlap.  Runs on hip_stream and returns after the enqueue. */
int nvfp4_transpose(const nvfp4_tensor *in, nvfp4_tensor *out, void *hip_stream);

/* As nvfp4_gemm, with C quantized in the epilogue instead of stored: the output of one layer leaves
 * the GEMM as the next layer's NVFP4 activation (the feed-forward chain that the pages' recipe runs
 * in FP4: hyper.ai (fr) story; aissential.tech article, Method).  out = Q(C), where C is the fp32
 * matrix nvfp4_gemm would store (c_dtype NVFP4_F32, same operands) and Q quantizes it row-wise in
 * 1D 16-element blocks along N with nearest-even rounding, exactly as nvfp4_quantize with flags 0,
 * except that the tensor scale is not derived from C: Q uses *out->tensor_scale, which the caller
 * writes beforehand (delayed scaling, e.g. from the amax of the previous call: this library's
 * reading, since the pages do not say how the tensor scale of a GEMM output is chosen).  Elements
 * beyond 6 times their block scale saturate to +-6 (block scales clamp at 448).
 * amax: nullable device float; if given, *amax = max(*amax, max |C|) when the GEMM completes (an
 * atomic maximum, so the caller zeroes it before the first call it should cover); turn it into the
 * next tensor scale with nvfp4_scale_from_amax.
 * out: [M x N] descriptor with flags 0, data 16-byte aligned, scales [M][N/16], tensor_scale the
 * input scale (device).  Supported when K % 256 == 0, K > 0 and both operands' scale arrays are
 * 16-byte aligned (else NVFP4_ERR_UNSUPPORTED); grouped operands as for nvfp4_gemm.  All buffers are
 * device memory owned by the caller; out must not overlap the inputs.  Runs on hip_stream. */
int nvfp4_gemm_nvfp4_out(const nvfp4_tensor *a, const nvfp4_tensor *b, nvfp4_tensor *out, float *amax,
                         int32_t num_groups, const int64_t *group_row_offsets, void *hip_stream);

/* *ts = RN(*amax / 2688) on the device: the format's FP32 tensor scale for a tensor maximum (amax
 * maps to 6 * 448, the largest E2M1 value times the largest E4M3 scale; aissential.tech article,
 * Summary).  amax and ts: device floats, 4-byte aligned.  Runs on hip_stream. */
int nvfp4_scale_from_amax(const float *amax, float *ts, void *hip_stream);

/* Weight-only 4-bit GEMM, bf16 activations x NVFP4 weights with FP32 accumulation (the W4A16 mode
 * that a serving stack falls back to where the hardware has no FP4 x FP4 product: hyper.ai (de)
 * story on the Nemotron 3 Ultra NVFP4 checkpoint, Hopper):
 *   C[i][j] = ts_b * sum_k a[i][k] * (q_b[j][k] * S_b(j,k)),
 * i.e. C = A * B^T with A [M x K] bf16 row-major (leading dimension lda elements) and B [N x K] = b
 * (N = b->rows, K = b->k, 1D or BLOCK2D scales).  Each weight element q*S is exact in bf16, each
 * product a*q*S exact in fp32, the K sum accumulates in fp32, and ts_b is applied once at the end.
 * a_dtype must be NVFP4_BF16 (else NVFP4_ERR_UNSUPPORTED).  c: device, [M x N] with leading
 * dimension ldc >= N, dtype NVFP4_F32 or NVFP4_BF16 (nearest-even).  K % 64 == 0 (else
 * NVFP4_ERR_SHAPE); a and b->data 16-byte aligned, lda * 2 a multiple of 16 bytes, b->scales
 * 4-byte aligned, c aligned to its element size (else NVFP4_ERR_ALIGN).  All buffers are device
 * memory owned by the caller; c must not overlap the inputs.  Runs on hip_stream and returns after
 * the enqueue. */
int nvfp4_gemm_w4a16(const void *a, int a_dtype, int64_t m, int64_t lda, const nvfp4_tensor *b, void *c,
                     int c_dtype, int64_t ldc, void *hip_stream);

/* Static, human-readable text for a status code. */
const char *nvfp4_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
