// nvfp4_api.cpp -- C ABI front end of libnvfp4.so: argument validation on the host, then the
// kernel launchers.  Validation never touches the GPU, so every error path can be exercised on a
// machine without one.
// The library is built with -fvisibility=hidden: only the declarations of the public header (which
// fix the visibility of the definitions below) are exported.
#pragma GCC visibility push(default)
#include "../../include/nvfp4.h"
#pragma GCC visibility pop

#include <hip/hip_runtime.h>

#include <mutex>

#include "nvfp4_internal.h"

namespace {

constexpr uint32_t kKnownFlags =
    NVFP4_COLWISE | NVFP4_BLOCK2D | NVFP4_SR | NVFP4_FOUR_OVER_SIX | NVFP4_TS_FOR_FOUR | NVFP4_SCALE_SEARCH;
constexpr int64_t kMaxIndex = int64_t(1) << 32;  // element / chunk counts are 32-bit in the kernels
constexpr int64_t kMaxQuantGroups = 65535;        // groups run along the grid's y dimension

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int dtype_size(int dt) { return dt == NVFP4_F32 ? 4 : (dt == NVFP4_BF16 ? 2 : 0); }

int check_flags(uint32_t flags, bool rht) {
  if (flags & ~kKnownFlags) return NVFP4_ERR_UNSUPPORTED;
  const bool sr = flags & NVFP4_SR, fos = flags & NVFP4_FOUR_OVER_SIX, b2d = flags & NVFP4_BLOCK2D;
  const bool search = flags & NVFP4_SCALE_SEARCH;
  if ((sr && (fos || search)) || (sr && b2d) || (fos && search) || (search && b2d) || (rht && b2d))
    return NVFP4_ERR_UNSUPPORTED;
  return NVFP4_OK;
}

// Shared validation of the quantize entry points; fills R, K.
int validate_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                      bool rht, const nvfp4_tensor *out, const void *workspace, int64_t *R, int64_t *K) {
  if (!out) return NVFP4_ERR_NULL;
  const int es = dtype_size(x_dtype);
  if (es == 0) return NVFP4_ERR_UNSUPPORTED;
  int st = check_flags(flags, rht);
  if (st != NVFP4_OK) return st;
  if (rows < 0 || cols < 0 || ldx < cols || ldx < 1) return NVFP4_ERR_SHAPE;
  const bool colwise = flags & NVFP4_COLWISE;
  *R = colwise ? cols : rows;
  *K = colwise ? rows : cols;
  if (*K % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((flags & NVFP4_BLOCK2D) && *R % 16 != 0) return NVFP4_ERR_SHAPE;
  if (colwise && cols % 8 != 0) return NVFP4_ERR_SHAPE;  // a lane reads 8 columns
  if (rows * cols >= kMaxIndex || rows * ldx >= kMaxIndex * 4) return NVFP4_ERR_SHAPE;
  if (out->rows != *R || out->k != *K || ((out->flags ^ flags) & NVFP4_BLOCK2D)) return NVFP4_ERR_SHAPE;
  if (*R == 0 || *K == 0) {
    if (!out->tensor_scale) return NVFP4_ERR_NULL;
    return NVFP4_OK;
  }
  if (!x || !out->data || !out->scales || !out->tensor_scale || !workspace) return NVFP4_ERR_NULL;
  if (!aligned16(x) || !aligned16(out->data) || !aligned16(workspace)) return NVFP4_ERR_ALIGN;
  if ((ldx * es) % 16 != 0) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

int run_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                 uint64_t seed, uint32_t stream_id, bool rht, uint64_t sign_seed, float *rht_out,
                 nvfp4_tensor *out, void *workspace, void *hip_stream, int64_t groups = 1, int64_t group_stride = 0) {
  int64_t R = 0, K = 0;
  int st = validate_quantize(x, x_dtype, rows, cols, ldx, flags, rht, out, workspace, &R, &K);
  if (st != NVFP4_OK) return st;
  if (rht_out && !aligned16(rht_out)) return NVFP4_ERR_ALIGN;
  nvfp4::QuantArgs a{};
  a.groups = groups;
  a.x_group_bytes = group_stride * dtype_size(x_dtype);
  a.x = x;
  a.dtype = x_dtype == NVFP4_BF16 ? 1 : 0;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.R = R;
  a.K = K;
  a.flags = flags;
  a.seed = seed;
  a.stream_id = stream_id;
  a.rht = rht;
  a.sign_word = 0;
  if (rht) {
    const uint32_t ctr[4] = {0u, 0u, 0u, 1u};
    const uint32_t key[2] = {static_cast<uint32_t>(sign_seed), static_cast<uint32_t>(sign_seed >> 32)};
    uint32_t w[4];
    nvfp4::philox4x32_10_host(ctr, key, w);
    a.sign_word = w[0] & 0xFFFFu;
  }
  a.rht_out = rht ? rht_out : nullptr;
  a.data = out->data;
  a.scales = out->scales;
  a.ts = out->tensor_scale;
  a.workspace = static_cast<uint32_t *>(workspace);
  a.stream = static_cast<hipStream_t>(hip_stream);
  return status_of(nvfp4::launch_quantize(a));
}

// Shared validation of the NVFP4 x NVFP4 GEMM entry points (shapes, groups, operand pointers).
int validate_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, int32_t num_groups, const int64_t *group_row_offsets) {
  if (!a || !b) return NVFP4_ERR_NULL;
  if (num_groups < 0 || (num_groups > 1 && !group_row_offsets)) return NVFP4_ERR_SHAPE;
  const int64_t M = a->rows, N = b->rows, K = a->k;
  if (M < 0 || N < 0 || K < 0 || b->k != K || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((a->flags & NVFP4_BLOCK2D) && M % 16 != 0) return NVFP4_ERR_SHAPE;
  if ((b->flags & NVFP4_BLOCK2D) && N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (M * K >= kMaxIndex || N * K >= kMaxIndex) return NVFP4_ERR_SHAPE;
  if (num_groups > 1 || group_row_offsets) {
    const int32_t G = num_groups < 1 ? 1 : num_groups;
    if (group_row_offsets[0] != 0 || group_row_offsets[G] != M) return NVFP4_ERR_SHAPE;
    for (int32_t g = 0; g < G; ++g)
      if (group_row_offsets[g + 1] < group_row_offsets[g]) return NVFP4_ERR_SHAPE;
  }
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a->tensor_scale || !b->tensor_scale) return NVFP4_ERR_NULL;
  if (K > 0) {  // (with K == 0 no code or scale is read)
    if (!a->data || !a->scales || !b->data || !b->scales) return NVFP4_ERR_NULL;
    if (!aligned16(a->data) || !aligned16(b->data)) return NVFP4_ERR_ALIGN;
  }
  return NVFP4_OK;
}

nvfp4::GemmArgs gemm_args(const nvfp4_tensor *a, const nvfp4_tensor *b, int32_t num_groups,
                          const int64_t *group_row_offsets, void *hip_stream) {
  nvfp4::GemmArgs g{};
  g.a_data = a->data;
  g.a_scales = a->scales;
  g.a_ts = a->tensor_scale;
  g.a_2d = (a->flags & NVFP4_BLOCK2D) != 0;
  g.b_data = b->data;
  g.b_scales = b->scales;
  g.b_ts = b->tensor_scale;
  g.b_2d = (b->flags & NVFP4_BLOCK2D) != 0;
  g.M = a->rows;
  g.N = b->rows;
  g.K = a->k;
  g.num_groups = num_groups < 1 ? 1 : num_groups;
  g.group_offsets = group_row_offsets;
  g.stream = static_cast<hipStream_t>(hip_stream);
  return g;
}

// ---- library-owned workspace for nvfp4_quantize_noalloc -----------------------------------------
// The amax pass's per-workgroup partial maxima live in this file-scope device array (one copy per
// GPU, held until the process ends) instead of a caller buffer.  Every call rewrites the slots it
// reads before reading them, so nothing needs clearing; calls that overlap on one GPU share it and
// race.  Host code never passes the array's name to a kernel (on the host it names a stand-in, not
// device memory): the device address comes from hipGetSymbolAddress, once per device with that
// device current, and is kept per device.
__device__ __align__(256) uint32_t scratch[nvfp4::kMaxParts];
constexpr size_t kScratchBytes = sizeof(uint32_t) * nvfp4::kMaxParts;
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call per device).
hipError_t scratch_address(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return *ptr != nullptr ? hipSuccess : hipErrorInvalidSymbol;
}

}  // namespace

namespace nvfp4 {
void philox4x32_10_host(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}
}  // namespace nvfp4

extern "C" {

size_t nvfp4_workspace_size(int64_t rows, int64_t cols, uint32_t flags) {
  (void)rows;
  (void)cols;
  (void)flags;
  return sizeof(uint32_t) * nvfp4::kMaxParts;
}

int nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                   uint64_t seed, uint32_t stream_id, nvfp4_tensor *out, void *workspace, void *hip_stream) {
  return run_quantize(x, x_dtype, rows, cols, ldx, flags, seed, stream_id, false, 0, nullptr, out, workspace,
                      hip_stream);
}

int nvfp4_quantize_noalloc(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                           uint64_t seed, uint32_t stream_id, nvfp4_tensor *out, void *hip_stream) {
  // the partial maxima never exceed the array (the pass-1 grid is capped at kMaxParts); checked so
  // that a larger need could not go unnoticed
  if (nvfp4_workspace_size(rows, cols, flags) > kScratchBytes) return NVFP4_ERR_SHAPE;
  int64_t R = 0, K = 0;
  static const uint32_t kAligned[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  // validate with a stand-in workspace pointer first: nothing touches the GPU on an invalid call
  int st = validate_quantize(x, x_dtype, rows, cols, ldx, flags, false, out, kAligned, &R, &K);
  if (st != NVFP4_OK) return st;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return NVFP4_ERR_HIP;
  return run_quantize(x, x_dtype, rows, cols, ldx, flags, seed, stream_id, false, 0, nullptr, out, ws, hip_stream);
}

int nvfp4_rht_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                       uint64_t seed, uint32_t stream_id, uint64_t sign_seed, float *rht_out, nvfp4_tensor *out,
                       void *workspace, void *hip_stream) {
  return run_quantize(x, x_dtype, rows, cols, ldx, flags, seed, stream_id, true, sign_seed, rht_out, out, workspace,
                      hip_stream);
}

int nvfp4_quantize_grouped(const void *x, int x_dtype, int64_t groups, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t group_stride, uint32_t flags, uint64_t seed, uint32_t stream_id,
                           nvfp4_tensor *out, void *workspace, void *hip_stream) {
  if (groups < 1 || groups > kMaxQuantGroups) return NVFP4_ERR_SHAPE;
  if (group_stride < 0 || (groups > 1 && group_stride > (kMaxIndex << 4) / (groups - 1))) return NVFP4_ERR_SHAPE;
  const int es = dtype_size(x_dtype);
  if (es != 0 && (group_stride * es) % 16 != 0) return NVFP4_ERR_ALIGN;
  return run_quantize(x, x_dtype, rows, cols, ldx, flags, seed, stream_id, false, 0, nullptr, out, workspace,
                      hip_stream, groups, group_stride);
}

int nvfp4_dequantize(const nvfp4_tensor *in, void *y, int y_dtype, int64_t ldy, void *hip_stream) {
  if (!in) return NVFP4_ERR_NULL;
  const int es = dtype_size(y_dtype);
  if (es == 0) return NVFP4_ERR_UNSUPPORTED;
  if (in->rows < 0 || in->k < 0 || in->k % 16 != 0 || ldy < in->k || ldy < 1) return NVFP4_ERR_SHAPE;
  if ((in->flags & NVFP4_BLOCK2D) && in->rows % 16 != 0) return NVFP4_ERR_SHAPE;
  if (in->rows * in->k >= kMaxIndex) return NVFP4_ERR_SHAPE;
  if (in->rows == 0 || in->k == 0) return NVFP4_OK;
  if (!in->data || !in->scales || !in->tensor_scale || !y) return NVFP4_ERR_NULL;
  if (!aligned16(in->data) || !aligned16(y) || (ldy * es) % 16 != 0) return NVFP4_ERR_ALIGN;
  nvfp4::DequantArgs a{in->data, in->scales, in->tensor_scale, in->rows, in->k,
                       (in->flags & NVFP4_BLOCK2D) != 0, y, y_dtype == NVFP4_BF16 ? 1 : 0, ldy,
                       static_cast<hipStream_t>(hip_stream)};
  return status_of(nvfp4::launch_dequantize(a));
}

int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype, int64_t ldc, int32_t num_groups,
               const int64_t *group_row_offsets, void *hip_stream) {
  if (!a || !b) return NVFP4_ERR_NULL;
  if (dtype_size(c_dtype) == 0) return NVFP4_ERR_UNSUPPORTED;
  int st = validate_gemm(a, b, num_groups, group_row_offsets);
  if (st != NVFP4_OK) return st;
  const int64_t M = a->rows, N = b->rows;
  if (ldc < N || ldc < 1 || M * ldc >= kMaxIndex * 4) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(c) & static_cast<uintptr_t>(dtype_size(c_dtype) - 1)) != 0) return NVFP4_ERR_ALIGN;
  nvfp4::GemmArgs g = gemm_args(a, b, num_groups, group_row_offsets, hip_stream);
  g.c = c;
  g.c_dtype = c_dtype == NVFP4_BF16 ? 1 : 0;
  g.ldc = ldc;
  return status_of(nvfp4::launch_gemm(g));
}

int nvfp4_gemm_nvfp4_out(const nvfp4_tensor *a, const nvfp4_tensor *b, nvfp4_tensor *out, float *amax,
                         int32_t num_groups, const int64_t *group_row_offsets, void *hip_stream) {
  if (!a || !b || !out) return NVFP4_ERR_NULL;
  int st = validate_gemm(a, b, num_groups, group_row_offsets);
  if (st != NVFP4_OK) return st;
  const int64_t M = a->rows, N = b->rows, K = a->k;
  // C is quantized in 16-column blocks along N: the output's K axis is N
  if (out->rows != M || out->k != N || N % 16 != 0) return NVFP4_ERR_SHAPE;
  if (out->flags != 0) return NVFP4_ERR_UNSUPPORTED;  // row-wise 1D blocks, nearest-even only
  if (M == 0 || N == 0) return NVFP4_OK;
  // the quantized epilogue lives in the pipelined kernel: whole pairs of 128-element K steps,
  // 16-byte aligned scale arrays
  if (K == 0 || K % 256 != 0 || (reinterpret_cast<uintptr_t>(a->scales) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(b->scales) & 15u) != 0)
    return NVFP4_ERR_UNSUPPORTED;
  if (!out->data || !out->scales || !out->tensor_scale) return NVFP4_ERR_NULL;
  if (!aligned16(out->data) || (amax && (reinterpret_cast<uintptr_t>(amax) & 3u) != 0)) return NVFP4_ERR_ALIGN;
  nvfp4::GemmArgs g = gemm_args(a, b, num_groups, group_row_offsets, hip_stream);
  g.c_dtype = 2;
  g.ldc = N;
  g.q_data = out->data;
  g.q_scales = out->scales;
  g.q_ts = out->tensor_scale;
  g.amax = amax;
  return status_of(nvfp4::launch_gemm(g));
}

int nvfp4_scale_from_amax(const float *amax, float *ts, void *hip_stream) {
  if (!amax || !ts) return NVFP4_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(amax) & 3u) != 0 || (reinterpret_cast<uintptr_t>(ts) & 3u) != 0) return NVFP4_ERR_ALIGN;
  return status_of(nvfp4::launch_scale_from_amax(amax, ts, static_cast<hipStream_t>(hip_stream)));
}

int nvfp4_gemm_w4a16(const void *a, int a_dtype, int64_t m, int64_t lda, const nvfp4_tensor *b, void *c,
                     int c_dtype, int64_t ldc, void *hip_stream) {
  if (!b) return NVFP4_ERR_NULL;
  if (a_dtype != NVFP4_BF16 || dtype_size(c_dtype) == 0) return NVFP4_ERR_UNSUPPORTED;
  const int64_t M = m, N = b->rows, K = b->k;
  if (M < 0 || N < 0 || K < 0 || K % 64 != 0 || lda < K || lda < 1 || ldc < N || ldc < 1) return NVFP4_ERR_SHAPE;
  if ((b->flags & NVFP4_BLOCK2D) && N % 16 != 0) return NVFP4_ERR_SHAPE;
  // byte offsets into A and B are 32-bit in the kernel
  if (M * lda >= kMaxIndex / 2 || N * K >= kMaxIndex || M * ldc >= kMaxIndex * 4) return NVFP4_ERR_SHAPE;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!b->tensor_scale || !c) return NVFP4_ERR_NULL;
  if (K > 0) {  // (with K == 0 nothing of A or B is read and C = 0)
    if (!a || !b->data || !b->scales) return NVFP4_ERR_NULL;
    if (!aligned16(a) || (lda * 2) % 16 != 0 || !aligned16(b->data) || (reinterpret_cast<uintptr_t>(b->scales) & 3u) != 0)
      return NVFP4_ERR_ALIGN;
  }
  if ((reinterpret_cast<uintptr_t>(c) & static_cast<uintptr_t>(dtype_size(c_dtype) - 1)) != 0) return NVFP4_ERR_ALIGN;
  nvfp4::W4A16Args w{};
  w.a = a;
  w.lda = lda;
  w.b_data = b->data;
  w.b_scales = b->scales;
  w.b_ts = b->tensor_scale;
  w.b_2d = (b->flags & NVFP4_BLOCK2D) != 0;
  w.M = M;
  w.N = N;
  w.K = K;
  w.c = c;
  w.c_dtype = c_dtype == NVFP4_BF16 ? 1 : 0;
  w.ldc = ldc;
  w.stream = static_cast<hipStream_t>(hip_stream);
  return status_of(nvfp4::launch_gemm_w4a16(w));
}

int nvfp4_transpose(const nvfp4_tensor *in, nvfp4_tensor *out, void *hip_stream) {
  if (!in || !out) return NVFP4_ERR_NULL;
  if (!(in->flags & NVFP4_BLOCK2D) || !(out->flags & NVFP4_BLOCK2D)) return NVFP4_ERR_UNSUPPORTED;
  const int64_t R = in->rows, K = in->k;
  if (R < 0 || K < 0 || R % 16 != 0 || K % 16 != 0 || out->rows != K || out->k != R) return NVFP4_ERR_SHAPE;
  if (R * K >= kMaxIndex) return NVFP4_ERR_SHAPE;
  if (!in->tensor_scale || !out->tensor_scale) return NVFP4_ERR_NULL;
  if (R > 0 && K > 0) {
    if (!in->data || !in->scales || !out->data || !out->scales) return NVFP4_ERR_NULL;
    if (!aligned16(in->data) || !aligned16(out->data)) return NVFP4_ERR_ALIGN;
  }
  nvfp4::TransposeLaunch t{};
  t.in_data = in->data;
  t.in_scales = in->scales;
  t.in_ts = in->tensor_scale;
  t.out_data = out->data;
  t.out_scales = out->scales;
  t.out_ts = out->tensor_scale;
  t.R = R;
  t.K = K;
  t.stream = static_cast<hipStream_t>(hip_stream);
  return status_of(nvfp4::launch_transpose(t));
}

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK: success";
    case NVFP4_ERR_NULL: return "NVFP4_ERR_NULL: a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE: invalid shape, leading dimension or descriptor";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN: pointer or leading dimension not 16-byte aligned";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED: unsupported dtype or flag combination";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP: a HIP launch failed";
    default: return "unknown nvfp4 status";
  }
}

}  // extern "C"
