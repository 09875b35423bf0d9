// nvfp4_internal.h -- private interface between the C-ABI front end (nvfp4_api.cpp) and the kernel
// launchers (*.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Upper bound on the number of amax-pass workgroups; the workspace holds one partial maximum each.
constexpr uint32_t kMaxParts = 4096;

struct QuantArgs {
  const void *x;
  int dtype;              // 0 = f32, 1 = bf16
  int64_t rows, cols, ldx;
  int64_t R, K;           // logical Y shape
  uint32_t flags;
  uint64_t seed;
  uint32_t stream_id;
  bool rht;
  uint32_t sign_word;
  float *rht_out;
  uint8_t *data;
  uint8_t *scales;
  float *ts;
  uint32_t *workspace;
  hipStream_t stream;
  int64_t groups = 1;         // equally shaped tensors quantized by one call (grid dimension y)
  int64_t x_group_bytes = 0;  // bytes between consecutive groups' inputs
};

struct DequantArgs {
  const uint8_t *data;
  const uint8_t *scales;
  const float *ts;
  int64_t R, K;
  bool block2d;
  void *y;
  int y_dtype;
  int64_t ldy;
  hipStream_t stream;
};

struct GemmArgs {
  const uint8_t *a_data, *a_scales;
  const float *a_ts;
  bool a_2d;
  const uint8_t *b_data, *b_scales;
  const float *b_ts;
  bool b_2d;
  int64_t M, N, K;
  void *c;
  int c_dtype;
  int64_t ldc;
  int32_t num_groups;
  const int64_t *group_offsets;  // host, num_groups + 1 (nullptr for a plain GEMM)
  hipStream_t stream;
  // c_dtype 2: C quantized to NVFP4 (1D, nearest-even) with tensor scale *q_ts; amax nullable
  uint8_t *q_data = nullptr, *q_scales = nullptr;
  const float *q_ts = nullptr;
  float *amax = nullptr;
};

struct W4A16Args {
  const void *a;  // bf16 [M x lda]
  int64_t lda;    // elements
  const uint8_t *b_data, *b_scales;
  const float *b_ts;
  bool b_2d;
  int64_t M, N, K;
  void *c;
  int c_dtype;
  int64_t ldc;
  hipStream_t stream;
};

struct TransposeLaunch {
  const uint8_t *in_data, *in_scales;
  const float *in_ts;
  uint8_t *out_data, *out_scales;
  float *out_ts;
  int64_t R, K;  // input logical shape
  hipStream_t stream;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_quantize(const QuantArgs &a);
hipError_t launch_dequantize(const DequantArgs &a);
hipError_t launch_gemm(const GemmArgs &a);
hipError_t launch_transpose(const TransposeLaunch &a);
hipError_t launch_gemm_w4a16(const W4A16Args &a);
hipError_t launch_scale_from_amax(const float *amax, float *ts, hipStream_t stream);

// Host copy of the Philox4x32-10 block function (for the RHT sign word).
void philox4x32_10_host(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

}  // namespace nvfp4
