// gemm.hip -- block-scaled NVFP4 x NVFP4 GEMM on the gfx950 matrix cores.
//
// C[i][j] = ts_a * ts_b * sum_k (q_a S_a)(q_b S_b).  The product of an E2M1 value (<= 2 significant
// bits, |q| <= 6) and an E4M3 scale (<= 4 significant bits, 2^-9 <= S <= 448) has at most 6
// significant bits and lies in [2^-10, 2688]: it is exact in fp16 (11 bits, normal from 2^-14).
// So every operand element is decoded exactly to fp16 with its block scale folded in, the matrix
// cores (v_mfma_f32_32x32x16_f16) form exact products and accumulate in fp32, and ts_a * ts_b is
// applied once in the epilogue.  The per-16-element scales never touch the accumulators.
//
// Both operands are K-major ([rows][K/2] packed codes).  In one MFMA a lane supplies 8 K-values of
// one row of A (row = lane & 31) and the same 8 K-positions of one row of B; any assignment of K
// positions to (lane half, slot) is valid as long as A and B use the same one.  A lane loads 16 B
// (32 codes) per row per 64-wide K step: lane half h takes codes [32h, 32h + 32) of the step, and
// MFMA m (m = 0..3) consumes its dword m.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr uint32_t kThreads = 256;
constexpr int kMaxGroupsPerLaunch = 128;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct GemmKArgs {
  const uint8_t *a_data, *a_scales;
  const float *a_ts;
  const uint8_t *b_data, *b_scales;
  const float *b_ts;
  int64_t N, K;
  uint8_t *c;
  int64_t ldc;
  int32_t groups;
  int32_t tiles_n;
  int64_t b_group_data;    // bytes between consecutive groups' B codes
  int64_t b_group_scales;  // bytes between consecutive groups' B scales
  int32_t group_base;      // index of the first group of this launch (for b offsets)
  int64_t row_begin[kMaxGroupsPerLaunch + 1];  // A rows of each group
  int32_t tile_begin[kMaxGroupsPerLaunch + 1]; // first tile of each group (prefix sums)
};

// E4M3 byte -> fp16 (exact: every E4M3 value is a normal fp16).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float f = e == 0 ? static_cast<float>(m) * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return static_cast<_Float16>(f);
}

// fp16 bits of the E2M1 value of a 4-bit code.
__device__ __forceinline__ uint32_t e2m1_f16_bits(uint32_t code) {
  uint32_t m = code & 7u;
  uint32_t mag = m >= 2u ? (m + 28u) << 9 : (m == 1u ? 0x3800u : 0u);
  return mag | ((code & 8u) << 12);
}

// 8 codes (one dword, code n at bits 4n) times scale S -> 8 exact fp16 values.
__device__ __forceinline__ half8 decode8(uint32_t w, _Float16 S) {
  half8 r;
  half2v s2 = {S, S};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = e2m1_f16_bits(w >> (8 * i)), hi = e2m1_f16_bits(w >> (8 * i + 4));
    half2v q = __builtin_bit_cast(half2v, lo | (hi << 16));
    half2v p = q * s2;
    r[2 * i] = p[0];
    r[2 * i + 1] = p[1];
  }
  return r;
}

template <bool OUT_BF16, bool A2D, bool B2D>
__global__ __launch_bounds__(kThreads) void gemm_simple_kernel(GemmKArgs p) {
  // tile -> (group, tile_m, tile_n)
  const int32_t tile = blockIdx.x;
  int32_t g = 0;
  while (g + 1 < p.groups && p.tile_begin[g + 1] <= tile) ++g;
  const int32_t local = tile - p.tile_begin[g];
  const int32_t tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int64_t row0 = p.row_begin[g], row1 = p.row_begin[g + 1];
  const uint8_t *b_data = p.b_data + static_cast<int64_t>(p.group_base + g) * p.b_group_data;
  const uint8_t *b_scales = p.b_scales + static_cast<int64_t>(p.group_base + g) * p.b_group_scales;
  const float ts = *p.a_ts * p.b_ts[p.group_base + g];

  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const int64_t KB = p.K / 16;
  const int64_t m_base = row0 + static_cast<int64_t>(tm) * 128 + (wave >> 1) * 64;
  const int64_t n_base = static_cast<int64_t>(tn) * 128 + (wave & 1) * 64;

  floatx16 acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][t][r] = 0.0f;

  for (int64_t k0 = 0; k0 < p.K; k0 += 64) {
    half8 af[2][4], bf[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t ra = m_base + 32 * s + l32;
      const int64_t rb = n_base + 32 * s + l32;
      const int64_t kc = k0 + 32 * h;  // first K of this lane's 32 codes
      uint4 wa = make_uint4(0, 0, 0, 0), wb = make_uint4(0, 0, 0, 0);
      uint32_t sa0 = 0, sa1 = 0, sb0 = 0, sb1 = 0;
      if (kc < p.K) {
        const bool full = kc + 32 <= p.K;  // K % 16 == 0: either 16 or 32 codes remain
        if (ra < row1) {
          const uint8_t *src = p.a_data + ra * (p.K / 2) + kc / 2;
          const uint2 lo = *reinterpret_cast<const uint2 *>(src);
          const uint2 hi = full ? *reinterpret_cast<const uint2 *>(src + 8) : make_uint2(0, 0);
          wa = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const uint8_t *sc = A2D ? p.a_scales + (ra / 16) * KB + kc / 16 : p.a_scales + ra * KB + kc / 16;
          sa0 = sc[0];
          sa1 = full ? sc[1] : 0u;
        }
        if (rb < p.N) {
          const uint8_t *src = b_data + rb * (p.K / 2) + kc / 2;
          const uint2 lo = *reinterpret_cast<const uint2 *>(src);
          const uint2 hi = full ? *reinterpret_cast<const uint2 *>(src + 8) : make_uint2(0, 0);
          wb = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const uint8_t *sc = B2D ? b_scales + (rb / 16) * KB + kc / 16 : b_scales + rb * KB + kc / 16;
          sb0 = sc[0];
          sb1 = full ? sc[1] : 0u;
        }
      }
      const _Float16 SA0 = e4m3_to_f16(sa0), SA1 = e4m3_to_f16(sa1);
      const _Float16 SB0 = e4m3_to_f16(sb0), SB1 = e4m3_to_f16(sb1);
      af[s][0] = decode8(wa.x, SA0);
      af[s][1] = decode8(wa.y, SA0);
      af[s][2] = decode8(wa.z, SA1);
      af[s][3] = decode8(wa.w, SA1);
      bf[s][0] = decode8(wb.x, SB0);
      bf[s][1] = decode8(wb.y, SB0);
      bf[s][2] = decode8(wb.z, SB1);
      bf[s][3] = decode8(wb.w, SB1);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[s][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s][m], bf[t][m], acc[s][t], 0, 0, 0);
  }

  // epilogue: lane holds column j = lane & 31, rows 8 * (r >> 2) + 4 * h + (r & 3)
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t col = n_base + 32 * t + l32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m_base + 32 * s + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row >= row1) continue;
        const float v = acc[s][t][r] * ts;
        if constexpr (OUT_BF16) {
          uint32_t b = __float_as_uint(v);
          uint16_t hb = static_cast<uint16_t>((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
          reinterpret_cast<uint16_t *>(p.c + row * p.ldc * 2)[col] = hb;
        } else {
          reinterpret_cast<float *>(p.c + row * p.ldc * 4)[col] = v;
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a) {
  const int32_t G = a.num_groups < 1 ? 1 : a.num_groups;
  const int64_t KB = a.K / 16;
  const int32_t tiles_n = static_cast<int32_t>((a.N + 127) / 128);
  for (int32_t g0 = 0; g0 < G; g0 += kMaxGroupsPerLaunch) {
    const int32_t ng = (G - g0) < kMaxGroupsPerLaunch ? (G - g0) : kMaxGroupsPerLaunch;
    GemmKArgs p{};
    p.a_data = a.a_data;
    p.a_scales = a.a_scales;
    p.a_ts = a.a_ts;
    p.b_data = a.b_data;
    p.b_scales = a.b_scales;
    p.b_ts = a.b_ts;
    p.N = a.N;
    p.K = a.K;
    p.c = static_cast<uint8_t *>(a.c);
    p.ldc = a.ldc;
    p.groups = ng;
    p.tiles_n = tiles_n;
    p.b_group_data = a.N * (a.K / 2);
    p.b_group_scales = a.b_2d ? (a.N / 16) * KB : a.N * KB;
    p.group_base = g0;
    int32_t tiles = 0;
    for (int32_t g = 0; g < ng; ++g) {
      const int64_t r0 = a.group_offsets ? a.group_offsets[g0 + g] : 0;
      const int64_t r1 = a.group_offsets ? a.group_offsets[g0 + g + 1] : a.M;
      p.row_begin[g] = r0;
      p.tile_begin[g] = tiles;
      tiles += static_cast<int32_t>(((r1 - r0) + 127) / 128) * tiles_n;
    }
    p.row_begin[ng] = a.group_offsets ? a.group_offsets[g0 + ng] : a.M;
    p.tile_begin[ng] = tiles;
    if (tiles == 0) continue;  // K == 0 still launches: the K loop is empty and C = 0
    const bool bf16 = a.c_dtype == 1;
#define NVFP4_GEMM(OB, A2, B2) \
  hipLaunchKernelGGL((gemm_simple_kernel<OB, A2, B2>), dim3(tiles), dim3(kThreads), 0, a.stream, p)
    if (bf16) {
      if (a.a_2d && a.b_2d) NVFP4_GEMM(true, true, true);
      else if (a.a_2d) NVFP4_GEMM(true, true, false);
      else if (a.b_2d) NVFP4_GEMM(true, false, true);
      else NVFP4_GEMM(true, false, false);
    } else {
      if (a.a_2d && a.b_2d) NVFP4_GEMM(false, true, true);
      else if (a.a_2d) NVFP4_GEMM(false, true, false);
      else if (a.b_2d) NVFP4_GEMM(false, false, true);
      else NVFP4_GEMM(false, false, false);
    }
#undef NVFP4_GEMM
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace nvfp4
