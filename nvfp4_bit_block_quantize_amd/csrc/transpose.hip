// transpose.hip -- transpose of an NVFP4 tensor with 16x16 block scales (HBM-bound).
//
// With 2D scaling a 16x16 tile of Y shares one scale and every element's code depends only on its
// value, the tile's scale and the tensor scale; transposing Y maps tiles onto tiles, so the
// quantization of Y^T is the quantization of Y with its codes and its scale grid transposed (no
// re-quantization).  This is how a weight quantized for the forward GEMM (K = in-features) serves
// the backward-data GEMM (K = out-features).
//
// A 256-thread workgroup moves a 64 x 64 tile of codes: each lane loads 16 codes (8 bytes) of one
// input row and spreads them as bytes into LDS, then gathers 16 codes of one input column (one
// output row) and stores them as 8 packed bytes.  The workgroup also moves the tile's 4 x 4 scale
// bytes.
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kT = 64;        // tile edge in elements
constexpr int kPitch = kT + 4; // LDS row pitch in bytes (one code per byte)

struct TransposeArgs {
  const uint8_t *in_data, *in_scales;
  const float *in_ts;
  uint8_t *out_data, *out_scales;
  float *out_ts;
  int64_t R, K;  // input logical shape (R, K multiples of 16)
};

__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs p) {
  __shared__ uint8_t tile[kT * kPitch];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kT, c0 = static_cast<int64_t>(blockIdx.x) * kT;
  const uint32_t t = threadIdx.x;
  // in: lane t takes input row r0 + t / 4, codes [16 (t % 4), 16 (t % 4) + 16) of the tile's columns
  {
    const uint32_t rr = t >> 2, q = t & 3;
    const int64_t r = r0 + rr, c = c0 + 16 * q;
    uint2 v = make_uint2(0, 0);
    if (r < p.R && c < p.K) v = *reinterpret_cast<const uint2 *>(p.in_data + r * (p.K / 2) + c / 2);
    uint8_t *dst = tile + rr * kPitch + 16 * q;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t w = b < 4 ? v.x : v.y;
      const uint32_t byte = (w >> (8 * (b & 3))) & 0xFFu;
      dst[2 * b] = static_cast<uint8_t>(byte & 15u);
      dst[2 * b + 1] = static_cast<uint8_t>(byte >> 4);
    }
  }
  // scales: the tile holds up to 4 x 4 blocks
  if (t < 16) {
    const int64_t br = r0 / 16 + (t >> 2), bc = c0 / 16 + (t & 3);
    if (br < p.R / 16 && bc < p.K / 16) p.out_scales[bc * (p.R / 16) + br] = p.in_scales[br * (p.K / 16) + bc];
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) *p.out_ts = *p.in_ts;
  __syncthreads();
  // out: lane t writes output row c0 + t / 4 (an input column), codes of input rows
  // [r0 + 16 (t % 4), r0 + 16 (t % 4) + 16)
  {
    const uint32_t cc = t >> 2, q = t & 3;
    const int64_t c = c0 + cc, r = r0 + 16 * q;
    if (c < p.K && r < p.R) {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t code = tile[(16 * q + e) * kPitch + cc];
        if (e < 8)
          w0 |= code << (4 * e);
        else
          w1 |= code << (4 * (e - 8));
      }
      *reinterpret_cast<uint2 *>(p.out_data + c * (p.R / 2) + r / 2) = make_uint2(w0, w1);
    }
  }
}

}  // namespace

hipError_t launch_transpose(const TransposeLaunch &a) {
  TransposeArgs p{a.in_data, a.in_scales, a.in_ts, a.out_data, a.out_scales, a.out_ts, a.R, a.K};
  // at least one workgroup: it copies the tensor scale also when the tensor is empty
  const uint32_t gx = a.K > 0 ? static_cast<uint32_t>((a.K + kT - 1) / kT) : 1u;
  const uint32_t gy = a.R > 0 ? static_cast<uint32_t>((a.R + kT - 1) / kT) : 1u;
  const dim3 grid(gx, gy);
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
