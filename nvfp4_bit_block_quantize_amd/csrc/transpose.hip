// transpose.hip -- transpose of an NVFP4 tensor with 16x16 block scales (HBM-bound).
//
// With 2D scaling a 16x16 tile of Y shares one scale and every element's code depends only on its
// value, the tile's scale and the tensor scale; transposing Y maps tiles onto tiles, so the
// quantization of Y^T is the quantization of Y with its codes and its scale grid transposed (no
// re-quantization).  This is how a weight quantized for the forward GEMM (K = in-features) serves
// the backward-data GEMM (K = out-features).
//
// A 256-thread workgroup moves a 128 x 128 tile of codes (8 KB each way) in three phases:
//   1. load: 8-byte pieces (16 codes) of the tile's 128 input rows into LDS, packed, rows 72 bytes
//      apart (8-byte global accesses: a row of K / 2 bytes is only 8-byte aligned);
//   2. transpose: lane (block row br, block column bc) reads one 8 x 8 block of codes as 8 dwords
//      (one per input row), transposes the nibble matrix in registers (three rounds of masked
//      swaps of 4-, 8- and 16-bit pieces between dword pairs) and writes the 8 dwords (one per
//      output row) into a second LDS tile, its dword column XOR-swizzled by bc so that a wave's
//      writes hit distinct banks;
//   3. store: 8-byte pieces of the 128 output rows to global memory.
// The workgroup also moves the tile's 8 x 8 scale bytes.  Each code moves by dword-wide LDS
// operations, where the earlier version moved it by two single-byte ones.
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr int kT = 128;       // tile edge in codes
constexpr int kPitch = 72;    // LDS row pitch in bytes (64 bytes of packed codes + 8)

struct TransposeArgs {
  const uint8_t *in_data, *in_scales;
  const float *in_ts;
  uint8_t *out_data, *out_scales;
  float *out_ts;
  int64_t R, K;  // input logical shape (R, K multiples of 16)
  // Paired order (a one-dimensional grid): a tile reads 64 bytes of each of its 128 input rows, half
  // of a 128-byte line, and the tile beside it reads the other half.  Workgroups L and L + 8 of
  // each 16 run on the same XCD (workgroup i runs on XCD i mod 8) and start together, so they take
  // the two tiles of a pair: each line is fetched into one L2 once instead of into two L2s.
  // gx = tile columns (even); 0 for the plain two-dimensional grid.
  uint32_t gx;
};

// 8 x 8 matrix of 4-bit codes, element (k, j) at bits 4j..4j+3 of d[k] -> element (k, j) at bits
// 4k..4k+3 of d[j]: the off-diagonal half-blocks of 1, 2 and then 4 nibbles are exchanged.
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t (&d)[8]) {
#pragma unroll
  for (int s = 1; s < 8; s <<= 1) {
    const uint32_t m = s == 1 ? 0x0F0F0F0Fu : (s == 2 ? 0x00FF00FFu : 0x0000FFFFu);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k & s) continue;
      const uint32_t t = ((d[k] >> (4 * s)) ^ d[k + s]) & m;
      d[k] ^= t << (4 * s);
      d[k + s] ^= t;
    }
  }
}

// W16: 16-byte global pieces (32 codes), for R and K multiples of 32 (rows 16-byte aligned); else
// 8-byte pieces (16 codes).
template <bool W16>
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t in_tile[kT * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t out_tile[kT * kPitch];
  uint32_t bx = blockIdx.x, by = blockIdx.y;
  if (p.gx != 0) {
    const uint32_t L = blockIdx.x, pair = (L >> 4) * 8u + (L & 7u), hp = p.gx / 2u;
    by = pair / hp;
    bx = 2u * (pair - by * hp) + ((L >> 3) & 1u);
  }
  const int64_t r0 = static_cast<int64_t>(by) * kT, c0 = static_cast<int64_t>(bx) * kT;
  const uint32_t t = threadIdx.x;
  const int64_t in_row = p.K / 2, out_row = p.R / 2;
  // 1. load: piece i of thread t is input row (t + 256 i) / PR, codes CP ((t + 256 i) % PR) .. + CP
  constexpr uint32_t CP = W16 ? 32 : 16, PR = kT / CP, NP = kT * PR / 256;  // codes per piece, pieces per row
#pragma unroll
  for (uint32_t i = 0; i < NP; ++i) {
    const uint32_t idx = t + 256u * i, rr = idx / PR, q = idx % PR;
    const int64_t r = r0 + rr, c = c0 + CP * q;
    uint8_t *const dst = in_tile + rr * kPitch + (CP / 2) * q;  // 8-byte aligned (the pitch is 72)
    if constexpr (W16) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < p.R && c < p.K) v = *reinterpret_cast<const uint4 *>(p.in_data + r * in_row + c / 2);
      reinterpret_cast<uint2 *>(dst)[0] = make_uint2(v.x, v.y);
      reinterpret_cast<uint2 *>(dst)[1] = make_uint2(v.z, v.w);
    } else {
      uint2 v = make_uint2(0, 0);
      if (r < p.R && c < p.K) v = *reinterpret_cast<const uint2 *>(p.in_data + r * in_row + c / 2);
      *reinterpret_cast<uint2 *>(dst) = v;
    }
  }
  // scales: the tile holds up to 8 x 8 blocks
  if (t < 64) {
    const int64_t br = r0 / 16 + (t >> 3), bc = c0 / 16 + (t & 7);
    if (br < p.R / 16 && bc < p.K / 16) p.out_scales[bc * (p.R / 16) + br] = p.in_scales[br * (p.K / 16) + bc];
  }
  if (bx == 0 && by == 0 && t == 0) *p.out_ts = *p.in_ts;
  __syncthreads();
  // 2. transpose: lane -> block (br, bc), bc = lane % 16, br = 4 wave + lane / 16
  {
    const uint32_t bc = t & 15u, br = t >> 4;
    uint32_t d[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = *reinterpret_cast<const uint32_t *>(in_tile + (8 * br + k) * kPitch + 4 * bc);
    transpose8x8_nibbles(d);
    const uint32_t col = br ^ (4u * ((bc >> 2) & 3u));  // swizzled dword column (keeps pairs together)
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t *>(out_tile + (8 * bc + j) * kPitch + 4 * col) = d[j];
  }
  __syncthreads();
  // 3. store: piece i of thread t is output row (t + 256 i) / PR (input column c0 + that), codes of
  // input rows r0 + CP ((t + 256 i) % PR) .. + CP (dword columns CP / 8 q .. of the swizzled tile: the
  // XOR by a multiple of 4 keeps a piece's 2 or 4 dwords contiguous)
#pragma unroll
  for (uint32_t i = 0; i < NP; ++i) {
    const uint32_t idx = t + 256u * i, orow = idx / PR, q = idx % PR;
    const int64_t c = c0 + orow, r = r0 + CP * q;
    const uint32_t col = ((CP / 8) * q) ^ (4u * ((orow >> 5) & 3u));
    const uint8_t *const src = out_tile + orow * kPitch + 4 * col;
    if constexpr (W16) {
      const uint2 lo = reinterpret_cast<const uint2 *>(src)[0], hi = reinterpret_cast<const uint2 *>(src)[1];
      if (c < p.K && r < p.R) *reinterpret_cast<uint4 *>(p.out_data + c * out_row + r / 2) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    } else {
      const uint2 v = *reinterpret_cast<const uint2 *>(src);
      if (c < p.K && r < p.R) *reinterpret_cast<uint2 *>(p.out_data + c * out_row + r / 2) = v;
    }
  }
}

}  // namespace

hipError_t launch_transpose(const TransposeLaunch &a) {
  TransposeArgs p{a.in_data, a.in_scales, a.in_ts, a.out_data, a.out_scales, a.out_ts, a.R, a.K, 0};
  // at least one workgroup: it copies the tensor scale also when the tensor is empty
  const uint32_t gx = a.K > 0 ? static_cast<uint32_t>((a.K + kT - 1) / kT) : 1u;
  const uint32_t gy = a.R > 0 ? static_cast<uint32_t>((a.R + kT - 1) / kT) : 1u;
  // paired order when the tiles fill whole groups of 16 workgroups in pairs of columns
  const uint64_t ntiles = static_cast<uint64_t>(gx) * gy;
  const bool paired = gx % 2 == 0 && ntiles % 16 == 0 && ntiles < (uint64_t(1) << 31);
  if (paired) p.gx = gx;
  const dim3 grid = paired ? dim3(static_cast<uint32_t>(ntiles)) : dim3(gx, gy);
  if (a.R % 32 == 0 && a.K % 32 == 0) hipLaunchKernelGGL(transpose_kernel<true>, grid, dim3(256), 0, a.stream, p);
  else hipLaunchKernelGGL(transpose_kernel<false>, grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
