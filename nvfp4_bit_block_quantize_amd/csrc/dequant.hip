// dequant.hip -- NVFP4 -> fp32 / bf16 decode (HBM-bound): y = RN(RN(q * S) * ts), then bf16
// nearest-even for a bf16 output.  Per 16-element block: 8 B of codes + 1 scale byte in, 64 B (fp32)
// or 32 B (bf16) out, split over 4 or 2 lanes.
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

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// A lane decodes E = 8 (bf16 out) or 4 (fp32 out) consecutive elements of one block, so every lane
// stores 16 contiguous bytes and a wave's store is one contiguous 1 KB run; the 16 / E lanes of a
// block share its scale byte.  q comes from v_cvt_scalef32_pk_f32_fp4 with scale 1.0 (two exact
// E2M1 values per instruction, code n of a byte at bits 4n).
template <bool BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DqArgs p) {
  constexpr uint32_t E = BF16 ? 8 : 4, LPB = 16 / E;
  const float ts = *p.ts;
  const uint32_t nlanes = p.nblocks * LPB;
  const uint32_t stride = gridDim.x * kThreads;
  const int64_t KB = p.K / 16;
  for (uint32_t u = blockIdx.x * kThreads + threadIdx.x; u < nlanes; u += stride) {
    const uint32_t b = u / LPB, part = u % LPB;
    const uint32_t r = fdiv(b, p.kb);
    const uint32_t kb = b - r * p.kb.d;
    const uint8_t *src = p.data + static_cast<int64_t>(r) * (p.K / 2) + 8 * kb + part * (E / 2);
    const uint32_t w = BF16 ? *reinterpret_cast<const uint32_t *>(src) : *reinterpret_cast<const uint16_t *>(src);
    const uint32_t sb = p.block2d ? p.scales[static_cast<int64_t>(r / 16) * KB + kb] : p.scales[static_cast<int64_t>(r) * KB + kb];
    const float S = e4m3_decode(sb);
    float v[E];
    const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    v[0] = (q0[0] * S) * ts;
    v[1] = (q0[1] * S) * ts;
    v[2] = (q1[0] * S) * ts;
    v[3] = (q1[1] * S) * ts;
    if constexpr (BF16) {
      const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
      const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      v[4] = (q2[0] * S) * ts;
      v[5] = (q2[1] * S) * ts;
      v[6] = (q3[0] * S) * ts;
      v[7] = (q3[1] * S) * ts;
    }
    uint8_t *dst = p.y + static_cast<int64_t>(r) * p.ldy_bytes +
                   static_cast<int64_t>(16 * kb + E * part) * (BF16 ? 2 : 4);
    if constexpr (BF16) {
      *reinterpret_cast<uint4 *>(dst) =
          make_uint4(bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16), bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16),
                     bf16_rne_bits(v[4]) | (bf16_rne_bits(v[5]) << 16), bf16_rne_bits(v[6]) | (bf16_rne_bits(v[7]) << 16));
    } else {
      *reinterpret_cast<float4 *>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const DequantArgs &a) {
  if (a.R == 0 || a.K == 0) return hipSuccess;
  DqArgs p{a.data, a.scales, a.ts, static_cast<uint32_t>(a.R * (a.K / 16)), make_fastdiv(static_cast<uint32_t>(a.K / 16)),
           a.K, a.block2d ? 1u : 0u, static_cast<uint8_t *>(a.y), a.ldy * (a.y_dtype == 1 ? 2 : 4)};
  const uint64_t lanes = static_cast<uint64_t>(p.nblocks) * (a.y_dtype == 1 ? 2 : 4);
  uint64_t want = (lanes + kThreads - 1) / kThreads;
  const uint32_t grid = static_cast<uint32_t>(want < (1u << 30) ? want : (1u << 30));
  if (a.y_dtype == 1)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(kThreads), 0, a.stream, p);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
