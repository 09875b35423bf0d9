// dequant.hip -- NVFP4 -> fp32 / bf16 decode (HBM-bound): y = RN(RN(q * S) * ts), then bf16
// nearest-even for a bf16 output.  One lane per 16-element block: 8 B of codes + 1 scale byte in,
// 64 B (fp32) or 32 B (bf16) out.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr uint32_t kThreads = 256;

struct DqArgs {
  const uint8_t *data;
  const uint8_t *scales;
  const float *ts;
  uint32_t nblocks;
  FastDiv kb;  // blocks per row
  int64_t K;
  uint32_t block2d;
  uint8_t *y;
  int64_t ldy_bytes;
};

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

__device__ __forceinline__ float e2m1_decode(uint32_t code) {
  uint32_t idx = code & 7u;
  uint32_t qb = idx >= 2u ? (idx + 252u) << 22 : (idx == 1u ? 0x3F000000u : 0u);
  return __uint_as_float(qb | ((code & 8u) << 28));
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DqArgs p) {
  const float ts = *p.ts;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < p.nblocks; b += stride) {
    const uint32_t r = fdiv(b, p.kb);
    const uint32_t kb = b - r * p.kb.d;
    const uint2 w = *reinterpret_cast<const uint2 *>(p.data + static_cast<int64_t>(r) * (p.K / 2) + 8 * kb);
    const int64_t KB = p.K / 16;
    const uint32_t sb = p.block2d ? p.scales[static_cast<int64_t>(r / 16) * KB + kb] : p.scales[static_cast<int64_t>(r) * KB + kb];
    const float S = e4m3_decode(sb);
    float v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      uint32_t code = ((t < 8 ? w.x : w.y) >> (4 * (t & 7))) & 15u;
      float q = e2m1_decode(code);
      float prod = q * S;
      v[t] = prod * ts;
    }
    uint8_t *dst = p.y + static_cast<int64_t>(r) * p.ldy_bytes + static_cast<int64_t>(kb) * 16 * (BF16 ? 2 : 4);
    if constexpr (BF16) {
      uint4 o[2];
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = bf16_rne_bits(v[2 * i]) | (bf16_rne_bits(v[2 * i + 1]) << 16);
      o[0] = make_uint4(h[0], h[1], h[2], h[3]);
      o[1] = make_uint4(h[4], h[5], h[6], h[7]);
      reinterpret_cast<uint4 *>(dst)[0] = o[0];
      reinterpret_cast<uint4 *>(dst)[1] = o[1];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        reinterpret_cast<float4 *>(dst)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const DequantArgs &a) {
  if (a.R == 0 || a.K == 0) return hipSuccess;
  DqArgs p{a.data, a.scales, a.ts, static_cast<uint32_t>(a.R * (a.K / 16)), make_fastdiv(static_cast<uint32_t>(a.K / 16)),
           a.K, a.block2d ? 1u : 0u, static_cast<uint8_t *>(a.y), a.ldy * (a.y_dtype == 1 ? 2 : 4)};
  uint64_t want = (p.nblocks + kThreads - 1) / kThreads;
  const uint32_t grid = static_cast<uint32_t>(want < (1u << 30) ? want : (1u << 30));
  if (a.y_dtype == 1)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(kThreads), 0, a.stream, p);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
