// gemm_common.hpp -- pieces shared by the MFMA GEMM kernels (NVFP4 x NVFP4 and bf16 x NVFP4): the
// 256 x 256 workgroup tile with four 128 x 128 wave quarters, direct global->LDS loads, the explicit
// waits and barrier of the LDS ring, the tile order, and the LDS-staged epilogue.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "nvfp4_device.hpp"

namespace nvfp4 {
namespace gemm {

constexpr uint32_t kThreads = 256;
constexpr int BM = 256, BN = 256;  // workgroup tile

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Direct global->LDS loads: lane l of the instruction writes its 16 (4) bytes at lds_base + 16 l
// (4 l); lds_base must be the same in every lane.
__device__ __forceinline__ void lds_load16(const uint8_t *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds((global_void *)g, (lds_void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_load4(const uint8_t *g, uint8_t *lds_base) {
  __builtin_amdgcn_global_load_lds((global_void *)g, (lds_void *)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(N) / lgkmcnt(0) only (the other counters left alone); gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that the compiler may not move memory accesses across; the caller has issued
// the waits that make its own LDS traffic complete.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pick(const uint4 &v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// fp32 -> bf16, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Map a workgroup id to a tile so that each of the 8 XCDs (workgroup i runs on XCD i % 8) owns a
// contiguous range of tiles.
__device__ __forceinline__ int32_t xcd_tile(int32_t wg, int32_t total) {
  if (total % 8 != 0) return wg;
  return (wg & 7) * (total >> 3) + (wg >> 3);
}

// Tile index -> (tile row, tile column), walking bands of 8 tile rows column by column, so that the
// tiles in flight together share their B columns and a few A rows in L2.
__device__ __forceinline__ void band_tile(int32_t local, int32_t tiles_n, int32_t tiles_m, int32_t &tm,
                                          int32_t &tn) {
  const int32_t band = 8;
  const int32_t per_band = band * tiles_n;
  const int32_t bi = local / per_band, rem = local - bi * per_band;
  const int32_t rows_in_band = min(band, tiles_m - bi * band);
  tn = rem / rows_in_band;
  tm = bi * band + (rem - tn * rows_in_band);
}

// C = acc * ts_a * ts_b per element: one multiply by ts_a * ts_b where that product is a normal fp32
// number (each element is then within one rounding of the exact product), else (acc * ts_a) * ts_b,
// so that a product of the two tensor scales that under- or overflows never reaches C.  (s1, s2) =
// (ts_a * ts_b, 1) or (ts_a, ts_b): the two-multiply form only where the product is not normal.
__device__ __forceinline__ void epilogue_scales(float ts_a, float ts_b, float &s1, float &s2, bool &one) {
  const float t = ts_a * ts_b;
  one = __builtin_isnormal(t);
  s1 = one ? t : ts_a;
  s2 = one ? 1.0f : ts_b;
}

// Epilogue of a 256 x 256 tile: C = acc * ts_a * ts_b, where acc[j][i] is the 32 x 32 product of the wave's
// B fragment j and A fragment i, so lane (h, l32) holds row l32 of tile (i, j), columns
// 8 (r >> 2) + 4 h + (r & 3).  Whole tiles go through LDS (smem, at least 4 x 32 x 512 bytes, no
// longer read by any wave's pending loads), 32 rows of the wave's quarter at a time, so that each
// store writes 16 consecutive bytes per lane and four (bf16) or two (fp32) complete 256 / 512-byte
// row segments per instruction; 16-byte chunk c of staged row r sits at c ^ (r mod chunks per row);
// rows at or beyond row_end are not written.  Tiles cut by N, or C without 16-byte aligned rows,
// take element stores.
// HALF: a 128 x 256 tile (rows at or beyond m0 + 128 are never stored) whose four waves each hold
// 128 rows x 64 columns: acc[j][i] for j < 2, wave w at columns 64 w.
template <bool HALF>
__device__ __forceinline__ uint32_t wave_row0(uint32_t wave) { return HALF ? 0u : (wave >> 1) * 128u; }
template <bool HALF>
__device__ __forceinline__ uint32_t wave_col0(uint32_t wave) { return HALF ? 64u * wave : (wave & 1) * 128u; }

// SPLIT (fp32 C of a full tile): the wave's 32-row pieces are staged one 64-column half at a time
// (8 KB per wave instead of 16), so that the staging fits the 32 KB ring stage a multi-tile
// workgroup hands the epilogue.
template <bool OUT_BF16, bool ONE, bool HALF, bool SPLIT>
__device__ __forceinline__ void store_c_rows(floatx16 (&acc)[4][4], uint8_t *smem, uint8_t *c, int64_t ldc,
                                             int64_t m0, int64_t n0, int64_t row_end, int64_t N, float ts_a,
                                             float ts_b, bool vec_store, uint32_t wave, uint32_t lane,
                                             bool settle) {
  // ONE: ts_a is the product of the two tensor scales (see epilogue_scales)
  auto sc = [&](float v) { return ONE ? v * ts_a : (v * ts_a) * ts_b; };
  constexpr int64_t ES = OUT_BF16 ? 2 : 4;
  constexpr int JN = HALF ? 2 : 4;  // B fragments (32 columns each) per wave
  // (lane through an opaque copy: in a kernel that runs several tiles, the epilogue's per-lane
  // addresses are then formed here and not hoisted out of the tile loop into spilled registers)
  asm volatile("" : "+v"(lane));
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t wm = wave_row0<HALF>(wave), wn = wave_col0<HALF>(wave);
  if (vec_store && n0 + BN <= N) {
    if (settle) {
      // all waves are done with the stages and the last (re-fetch) loads have landed
      wait_vmcnt<0>();
      wait_lgkmcnt0();
      lds_barrier();
    }
    constexpr int JH = (SPLIT && !OUT_BF16 && !HALF) ? 2 : 1;  // column passes
    constexpr int JP = JN / JH;                                  // B fragments per pass
    constexpr uint32_t ROWB = 32 * JP * ES, NCH = ROWB / 16;
    uint8_t *const region = smem + wave * (32 * ROWB);
    uint8_t *const gbase = c + ((m0 + wm) * ldc + n0 + wn) * ES;
    int64_t rows_left = row_end - (m0 + wm);  // rows of the wave's quarter that exist
    if (HALF && rows_left > 128) rows_left = 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (32 * i >= rows_left) break;  // wave-uniform
#pragma unroll
      for (int jh = 0; jh < JH; ++jh) {
#pragma unroll
        for (int jj = 0; jj < JP; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = JP * jh + jj;
            const float v0 = sc(acc[j][i][4 * q]), v1 = sc(acc[j][i][4 * q + 1]);
            const float v2 = sc(acc[j][i][4 * q + 2]), v3 = sc(acc[j][i][4 * q + 3]);
            if constexpr (OUT_BF16) {
              // v_cvt_pk_bf16_f32: nearest-even, as bf16_rne
              const bf16x2v lo = __builtin_convertvector((float2v){v0, v1}, bf16x2v);
              const bf16x2v hi = __builtin_convertvector((float2v){v2, v3}, bf16x2v);
              const uint32_t ch = 4 * jj + q;
              *reinterpret_cast<uint2 *>(region + l32 * ROWB + ((ch ^ (l32 & (NCH - 1))) * 16 + 8 * h)) =
                  make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
            } else {
              const uint32_t ch = 8 * jj + 2 * q + h;
              *reinterpret_cast<float4 *>(region + l32 * ROWB + (ch ^ (l32 & (NCH - 1))) * 16) =
                  make_float4(v0, v1, v2, v3);
            }
          }
        // the wave reads back its own rows (LDS accesses of one wave complete in order, so the next
        // pass's writes follow these reads)
#pragma unroll
        for (uint32_t t = 0; t < 32 * NCH / 64; ++t) {
          const uint32_t row = t * (64 / NCH) + lane / NCH, u = lane % NCH;
          const uint4 v = *reinterpret_cast<const uint4 *>(region + row * ROWB + ((u ^ (row & (NCH - 1))) * 16));
          if (32 * i + row < rows_left)
            *reinterpret_cast<uint4 *>(gbase + (32 * i + row) * ldc * ES + jh * ROWB + u * 16) = v;
        }
      }
    }
  } else {
    const int64_t row0 = m0 + wm + l32, col0 = n0 + wn + 4 * h;
    const int64_t row_stop = HALF && row_end > m0 + 128 ? m0 + 128 : row_end;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + 32 * i;
      if (row >= row_stop) continue;
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t col = col0 + 32 * j + 8 * (r >> 2) + (r & 3);
          if (col >= N) continue;
          const float v = sc(acc[j][i][r]);
          if constexpr (OUT_BF16)
            reinterpret_cast<uint16_t *>(c + row * ldc * 2)[col] = static_cast<uint16_t>(bf16_rne(v));
          else
            reinterpret_cast<float *>(c + row * ldc * 4)[col] = v;
        }
    }
  }
}

// settle = false: smem is a region (waves x 32 x 128 B per element byte) that no wave reads and no
// load in flight writes, so the staging neither waits for loads nor needs a barrier first.
template <bool OUT_BF16, bool HALF = false, bool SPLIT = false>
__device__ __forceinline__ void store_c_tile(floatx16 (&acc)[4][4], uint8_t *smem, uint8_t *c, int64_t ldc,
                                             int64_t m0, int64_t n0, int64_t row_end, int64_t N, float ts_a,
                                             float ts_b, bool vec_store, uint32_t wave, uint32_t lane,
                                             bool settle = true) {
  float s1, s2;
  bool one;
  epilogue_scales(ts_a, ts_b, s1, s2, one);
  if (one)
    store_c_rows<OUT_BF16, true, HALF, SPLIT>(acc, smem, c, ldc, m0, n0, row_end, N, s1, s2, vec_store, wave, lane, settle);
  else
    store_c_rows<OUT_BF16, false, HALF, SPLIT>(acc, smem, c, ldc, m0, n0, row_end, N, s1, s2, vec_store, wave, lane, settle);
}

// Quantized epilogue: C = acc * ts_a * ts_b (the fp32 values store_c_tile would write) is quantized
// row-wise in 16-column blocks, nearest-even, with the given tensor scale ts_q: codes to
// q_data [rows][N / 2], scale bytes to q_scales [rows][N / 16] (N % 16 == 0).  Each wave stages
// 32 rows x 128 columns of fp32 through LDS (16-byte chunk c of row r at c ^ (r & 31)); lane
// (row 8 t + (l >> 3), block l & 7) encodes one block per t, so eight lanes write a row's 64 bytes
// of codes.  Returns the lane's maximum |C| over the blocks it stored.
__device__ __forceinline__ float store_q_tile(floatx16 (&acc)[4][4], uint8_t *smem, uint8_t *q_data, uint8_t *q_scales,
                                              int64_t N, int64_t m0, int64_t n0, int64_t row_end, float ts_a,
                                              float ts_b, float ts_q, uint32_t wave, uint32_t lane) {
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
  // all waves are done with the stages and the last (re-fetch) loads have landed
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  lds_barrier();
  constexpr uint32_t ROWB = 512;  // 128 fp32
  uint8_t *const region = smem + wave * (32 * ROWB);
  const int64_t qrow = N / 2, srow = N / 16;
  float amax = 0.0f;
  float s1, s2;  // (v * s1) * s2 is the value store_c_tile writes (v * ts_a * ts_b when s2 == 1)
  bool one;
  epilogue_scales(ts_a, ts_b, s1, s2, one);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t ch = 8 * j + 2 * q + h;
        *reinterpret_cast<float4 *>(region + l32 * ROWB + (ch ^ (l32 & 31)) * 16) =
            make_float4((acc[j][i][4 * q] * s1) * s2, (acc[j][i][4 * q + 1] * s1) * s2,
                        (acc[j][i][4 * q + 2] * s1) * s2, (acc[j][i][4 * q + 3] * s1) * s2);
      }
    // the wave reads back its own rows (LDS accesses of one wave complete in order)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t row = 8 * t + (lane >> 3), blk = lane & 7u;
      float y[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 v = *reinterpret_cast<const float4 *>(region + row * ROWB + (((4 * blk + u) ^ (row & 31)) * 16));
        y[4 * u] = v.x;
        y[4 * u + 1] = v.y;
        y[4 * u + 2] = v.z;
        y[4 * u + 3] = v.w;
      }
      const int64_t grow = m0 + wm + 32 * i + row, gcol = n0 + wn + 16 * blk;
      if (grow < row_end && gcol < N) {
        const float ab = block_absmax(y);
        amax = fmaxf(amax, ab);
        uint32_t sbyte, w0, w1;
        encode_block_rne(y, ab, ts_q, sbyte, w0, w1);
        *reinterpret_cast<uint2 *>(q_data + grow * qrow + gcol / 2) = make_uint2(w0, w1);
        q_scales[grow * srow + gcol / 16] = static_cast<uint8_t>(sbyte);
      }
    }
  }
  return amax;
}

}  // namespace gemm
}  // namespace nvfp4
