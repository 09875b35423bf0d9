// gemm_kernels.hpp -- the block-scaled NVFP4 x NVFP4 GEMM kernels (templates) and their launcher.
// Each (output type, A scale layout, B scale layout) combination is instantiated in its own
// translation unit (gemm_variant.hip, compiled once per combination), so that the heavily unrolled
// instances compile in parallel; gemm.hip dispatches to them.
//
// C[i][j] = ts_a * ts_b * sum_k (q_a S_a)(q_b S_b).  The product of an E2M1 value (<= 2 significant
// bits, |q| <= 6) and an E4M3 scale (<= 4 significant bits, 2^-9 <= S <= 448) has at most 6
// significant bits and lies in [2^-10, 2688]: it is exact in fp16 (11 bits, normal from 2^-14).
// So every operand element is decoded exactly to fp16 with its block scale folded in, the matrix
// cores (v_mfma_f32_32x32x16_f16) form exact products and accumulate in fp32, and ts_a * ts_b is
// applied once in the epilogue.  The per-16-element scales never touch the accumulators.
//
// Decode: v_cvt_scalef32_pk_f16_fp4 with scale 1.0 turns two codes into two exact fp16 values
// (the instruction applies only the power-of-two part of its scale operand, so the E4M3 scale is
// applied separately), then one v_pk_mul_f16 by (S, S): about one VALU op per element.
//
// Tiling: a 256-thread workgroup computes a 256 x 256 tile of C; its four waves each own a
// 128 x 128 quarter (4 x 4 MFMA tiles of 32 x 32, 256 fp32 accumulators per lane).  K advances 128
// codes (64 bytes per row) per step through a double-buffered LDS stage:
//   codes   [256 rows][64 B] per operand, 16-byte chunk c of row r at chunk c ^ ((r >> 1) & 3)
//   scales  [256 rows][8 blocks] as fp16 pairs (S, S), converted once per workgroup while staging,
//           16-byte half h of row r at h ^ ((r >> 2) & 1)
// (the XOR swizzles give conflict-free ds_read_b128 for eight consecutive rows).  Within a step,
// lane half h of a 32-row MFMA fragment takes codes [64h, 64h + 64) of the step and MFMA m = 0..7
// consumes its dword m; A and B use the same K assignment, which is all the product needs.
#pragma once

#include "gemm_common.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace gemm {

constexpr int kMaxGroupsPerLaunch = 128;
constexpr int BKB = 64;            // bytes of codes per row per K step (128 codes)
constexpr int kCodeBytes = BM * BKB;        // one operand's codes per stage (16 KB)
constexpr int kScaleBytes = BM * 8 * 4;     // one operand's fp16-pair scales per stage (8 KB)
constexpr int kStageBytes = 2 * kCodeBytes + 2 * kScaleBytes;  // A + B

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

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
  int32_t total_tiles;
  int64_t b_group_data;    // bytes between consecutive groups' B codes
  int64_t b_group_scales;  // bytes between consecutive groups' B scales
  int32_t group_base;      // index of the first group of this launch (for b offsets)
  int32_t vec_store;       // C and its rows are 16-byte aligned (row-segment stores)
  uint8_t *q_data, *q_scales;  // quantized output (NVFP4 out only)
  const float *q_ts;           // its tensor scale (input)
  float *amax;                 // nullable: max |C| is folded into *amax
  int64_t row_begin[kMaxGroupsPerLaunch + 1];  // first A row of each group's tiles in this launch
  int64_t row_end[kMaxGroupsPerLaunch];        // end of each group's A rows
  int32_t tile_begin[kMaxGroupsPerLaunch + 1]; // first tile of each group (prefix sums)
};

// E4M3 byte b -> the fp16 pair (S, S) (the hardware fp8 decode is exact: every E4M3 value is a
// normal fp16 number).
__device__ __forceinline__ uint32_t scale_pair(uint32_t b) {
  half2v h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b * 0x101u, 1.0f, false);
  return __builtin_bit_cast(uint32_t, h);
}

// 8 codes (one dword, code n at bits 4n) times (S, S) -> 8 exact fp16 values.
__device__ __forceinline__ half8 decode8(uint32_t w, uint32_t s2bits) {
  const half2v s2 = __builtin_bit_cast(half2v, s2bits);
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Per-thread staging registers for one K step of one operand: 4 x 16 B of codes, 8 scale bytes,
// and which of the four code chunks / the scale row lie inside the operand.
struct Stage {
  uint4 code[4];
  uint32_t sc_lo, sc_hi;
  uint32_t valid;  // bits 0..3: code chunks, bit 4: scale row
};

// Global -> registers for rows [row0, row0 + 256) of an operand with valid rows below rows_end.
// FULL (K % 128 == 0): every step is whole, so the loads are unconditional: out-of-range rows read
// a clamped (valid) row and are zeroed when staged into LDS; no branch separates a load from its
// use, so all loads of a step stay in flight together.
template <bool B2D, bool FULL>
__device__ __forceinline__ void load_stage(Stage &st, const uint8_t *__restrict__ data,
                                           const uint8_t *__restrict__ scales, int64_t row0, int64_t rows_end,
                                           int64_t K, int64_t kt) {
  const int64_t row_bytes = K / 2, KB = K / 16;
  const int64_t kb0 = kt * BKB;  // byte offset of this step within a row
  st.valid = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = threadIdx.x + kThreads * i;
    const int64_t r = row0 + (c >> 2);
    const int64_t off = kb0 + 16 * (c & 3);
    if constexpr (FULL) {
      const int64_t rc = r < rows_end ? r : rows_end - 1;
      st.code[i] = *reinterpret_cast<const uint4 *>(data + rc * row_bytes + off);
      st.valid |= (r < rows_end ? 1u : 0u) << i;
    } else {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < rows_end) {
        const uint8_t *src = data + r * row_bytes + off;
        if (off + 16 <= row_bytes) {
          v = *reinterpret_cast<const uint4 *>(src);
        } else if (off + 8 <= row_bytes) {
          const uint2 h = *reinterpret_cast<const uint2 *>(src);
          v = make_uint4(h.x, h.y, 0, 0);
        }
      }
      st.code[i] = v;
      st.valid |= 1u << i;
    }
  }
  // scales: thread t -> row t, 8 bytes = blocks [8 kt, 8 kt + 8)
  const int64_t r = row0 + threadIdx.x;
  if constexpr (FULL) {
    const int64_t rc = r < rows_end ? r : rows_end - 1;
    const uint2 v = *reinterpret_cast<const uint2 *>(scales + (B2D ? (rc / 16) * KB : rc * KB) + 8 * kt);
    st.sc_lo = v.x;
    st.sc_hi = v.y;
    st.valid |= (r < rows_end ? 1u : 0u) << 4;
  } else {
    uint32_t lo = 0, hi = 0;
    if (r < rows_end) {
      const uint8_t *src = scales + (B2D ? (r / 16) * KB : r * KB) + 8 * kt;
      const int64_t nb = KB - 8 * kt;  // blocks left in the row
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b = j < nb ? src[j] : 0u;
        if (j < 4)
          lo |= b << (8 * j);
        else
          hi |= b << (8 * (j - 4));
      }
    }
    st.sc_lo = lo;
    st.sc_hi = hi;
    st.valid |= 1u << 4;
  }
}

// Registers -> LDS stage (codes swizzled, scales converted to fp16 pairs).
__device__ __forceinline__ void store_stage(const Stage &st, uint8_t *codes, uint8_t *scales) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t c = threadIdx.x + kThreads * i;
    const uint32_t r = c >> 2, ch = c & 3;
    const uint4 v = ((st.valid >> i) & 1u) ? st.code[i] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4 *>(codes + r * BKB + 16 * (ch ^ ((r >> 1) & 3))) = v;
  }
  const uint32_t r = threadIdx.x;
  const uint32_t lo = ((st.valid >> 4) & 1u) ? st.sc_lo : 0u, hi = ((st.valid >> 4) & 1u) ? st.sc_hi : 0u;
  uint4 h0, h1;  // blocks 0..3 and 4..7
  h0.x = scale_pair(lo & 0xFF);
  h0.y = scale_pair((lo >> 8) & 0xFF);
  h0.z = scale_pair((lo >> 16) & 0xFF);
  h0.w = scale_pair(lo >> 24);
  h1.x = scale_pair(hi & 0xFF);
  h1.y = scale_pair((hi >> 8) & 0xFF);
  h1.z = scale_pair((hi >> 16) & 0xFF);
  h1.w = scale_pair(hi >> 24);
  const uint32_t sw = (r >> 2) & 1;
  *reinterpret_cast<uint4 *>(scales + r * 32 + 16 * sw) = h0;
  *reinterpret_cast<uint4 *>(scales + r * 32 + 16 * (1 ^ sw)) = h1;
}

template <bool OUT_BF16, bool A2D, bool B2D, bool FULL>
__global__ __attribute__((visibility("hidden"))) __launch_bounds__(kThreads, 1) void gemm_kernel(GemmKArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];

  // ---- tile -> (group, tile_m, tile_n) ----
  const int32_t tile = xcd_tile(blockIdx.x, p.total_tiles);
  int32_t g = 0;
  while (g + 1 < p.groups && p.tile_begin[g + 1] <= tile) ++g;
  const int32_t local = tile - p.tile_begin[g];
  const int32_t tiles_m_g = (p.tile_begin[g + 1] - p.tile_begin[g]) / p.tiles_n;
  int32_t tm, tn;
  band_tile(local, p.tiles_n, tiles_m_g, tm, tn);
  const int64_t row_end = p.row_end[g];
  const uint8_t *b_data = p.b_data + static_cast<int64_t>(p.group_base + g) * p.b_group_data;
  const uint8_t *b_scales = p.b_scales + static_cast<int64_t>(p.group_base + g) * p.b_group_scales;
  const float ts_a = *p.a_ts, ts_b = p.b_ts[p.group_base + g];

  const int64_t m0 = p.row_begin[g] + static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;
  const int64_t KT = (p.K + 127) / 128;

  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t wm = (wave >> 1) * 128, wn = (wave & 1) * 128;  // wave quarter within the tile

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Stage sa, sb;
  if (KT > 0) {
    load_stage<A2D, FULL>(sa, p.a_data, p.a_scales, m0, row_end, p.K, 0);
    load_stage<B2D, FULL>(sb, b_data, b_scales, n0, p.N, p.K, 0);
    store_stage(sa, smem, smem + 2 * kCodeBytes);
    store_stage(sb, smem + kCodeBytes, smem + 2 * kCodeBytes + kScaleBytes);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      load_stage<A2D, FULL>(sa, p.a_data, p.a_scales, m0, row_end, p.K, kt + 1);
      load_stage<B2D, FULL>(sb, b_data, b_scales, n0, p.N, p.K, kt + 1);
    }
    const uint8_t *stage = smem + (kt & 1) * kStageBytes;
    const uint8_t *a_codes = stage, *b_codes = stage + kCodeBytes;
    const uint8_t *a_sc = stage + 2 * kCodeBytes, *b_sc = stage + 2 * kCodeBytes + kScaleBytes;

    // fragments: 4 A and 4 B row groups of 32; per lane 64 codes (two 16 B chunks) and 4 scales
    uint4 ac[4][2], bc[4][2], as4[4], bs4[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t ra = wm + 32 * f + l32, rb = wn + 32 * f + l32;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t ch = 2 * h + q;
        ac[f][q] = *reinterpret_cast<const uint4 *>(a_codes + ra * BKB + 16 * (ch ^ ((ra >> 1) & 3)));
        bc[f][q] = *reinterpret_cast<const uint4 *>(b_codes + rb * BKB + 16 * (ch ^ ((rb >> 1) & 3)));
      }
      as4[f] = *reinterpret_cast<const uint4 *>(a_sc + ra * 32 + 16 * (h ^ ((ra >> 2) & 1)));
      bs4[f] = *reinterpret_cast<const uint4 *>(b_sc + rb * 32 + 16 * (h ^ ((rb >> 2) & 1)));
    }
    // decode sub-step m + 1 while the 16 MFMAs of sub-step m run; the scheduling barriers ask for
    // one MFMA followed by four decode instructions, so the matrix pipe never waits on a long run of
    // VALU work (one wave per SIMD issues in order)
    auto decode_step = [&](int m, half8 (&af)[4], half8 (&bf)[4]) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint4 &wa = ac[f][m >> 2];
        const uint4 &wb = bc[f][m >> 2];
        const uint32_t da = (m & 3) == 0 ? wa.x : (m & 3) == 1 ? wa.y : (m & 3) == 2 ? wa.z : wa.w;
        const uint32_t db = (m & 3) == 0 ? wb.x : (m & 3) == 1 ? wb.y : (m & 3) == 2 ? wb.z : wb.w;
        const uint32_t sa2 = (m >> 1) == 0 ? as4[f].x : (m >> 1) == 1 ? as4[f].y : (m >> 1) == 2 ? as4[f].z : as4[f].w;
        const uint32_t sb2 = (m >> 1) == 0 ? bs4[f].x : (m >> 1) == 1 ? bs4[f].y : (m >> 1) == 2 ? bs4[f].z : bs4[f].w;
        af[f] = decode8(da, sa2);
        bf[f] = decode8(db, sb2);
      }
    };
    half8 afc[4], bfc[4];
    decode_step(0, afc, bfc);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      half8 afn[4], bfn[4];
      if (m < 7) decode_step(m + 1, afn, bfn);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afc[i], bfc[j], acc[i][j], 0, 0, 0);
      if (m < 7) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          afc[f] = afn[f];
          bfc[f] = bfn[f];
        }
      }
    }
    if (more) {
      uint8_t *nxt = smem + ((kt + 1) & 1) * kStageBytes;
      store_stage(sa, nxt, nxt + 2 * kCodeBytes);
      store_stage(sb, nxt + kCodeBytes, nxt + 2 * kCodeBytes + kScaleBytes);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds column l32 of each 32 x 32 tile, rows 8 * (r >> 2) + 4 * h + (r & 3)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn + 32 * j + l32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row >= row_end) continue;
        const float v = (acc[i][j][r] * ts_a) * ts_b;
        if constexpr (OUT_BF16) {
          const uint32_t b = __float_as_uint(v);
          reinterpret_cast<uint16_t *>(p.c + row * p.ldc * 2)[col] =
              static_cast<uint16_t>((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        } else {
          reinterpret_cast<float *>(p.c + row * p.ldc * 4)[col] = v;
        }
      }
    }
}


// ---- pipelined kernel (K % 128 == 0) ----------------------------------------------------------------
// Same tile and wave layout as gemm_kernel.  The operands reach LDS through direct global->LDS loads
// (global_load_lds: lane l of an instruction writes 16 B at the LDS base + 16 l, so the swizzle is
// applied by choosing which global chunk each lane fetches) into a ring of three stages, two K steps
// ahead of the math.  A K step takes its three stages (current, next, refill target) as __restrict__
// pointers, so the compiler knows that a fragment read does not alias the direct loads in flight to
// another stage and does not stall on them; the explicit waits before the step's barrier are what
// order the loads of one step before the reads of the next (for this wave and, through the barrier,
// for the others).
// One barrier per step, after sub-step 4: by then every wave holds the step's codes in registers;
// after it the next step's first codes and scales are read, and decoded under the last MFMAs.
// The MFMA takes the B fragment as its first operand, so that a lane's accumulators hold four
// consecutive columns of one row of C (staged through LDS for whole-row-segment stores).
// Rows beyond the operand read a clamped valid row: their products reach only outputs that are never
// stored.  Steps beyond K re-fetch the last step into a stage that is never consumed.
// PAIRED (an even number of K steps, 16-byte aligned scale rows): block scales travel two K steps
// at a time.  A row's 16 scale bytes of steps 2P and 2P + 1 are contiguous in memory, so one 16-byte
// direct load per lane moves 64 rows' worth.  They live in a ring of three slots of their own (A
// [256 rows][16 B], then B); pair P is loaded during steps 2P - 4 (A) and 2P - 3 (B), one load per
// wave each, so every step issues the same nine loads per lane (eight for codes) and the waits are
// constants.  Pair P's slot is reused for pair P + 3, first written in step 2P + 2, after the barrier
// of step 2P + 1 that follows the last read of pair P.
// Otherwise each stage carries its step's scales ([256 rows][8 B] per operand, dword loads: waves
// 0-1 A's, 2-3 B's), twelve loads per lane per step.
constexpr int kPA = 0, kPB = 16384, kPCodes = 32768;  // code stage layout (bytes)
constexpr int kPSlot = 8192;                          // PAIRED: one scale slot, A then B, 4 KB each
constexpr int kPSA = 32768, kPSB = 34816;             // otherwise: the stage's scales
template <bool PAIRED>
struct PipeLayout {
  static constexpr int kStage = PAIRED ? kPCodes : kPCodes + 4096;
  static constexpr int kScales = 3 * kStage;  // PAIRED: the three scale slots follow the stages
  static constexpr int kBytes = 3 * kStage + (PAIRED ? 3 * kPSlot : 0);
  static constexpr int kLoadsPerStage = PAIRED ? 9 : 12;  // direct loads issued per lane per step
};

// Chunk c (16 B) of tile row r is stored at position c ^ swz(r) of its 64-byte row: 8 or 16
// consecutive rows reading the same chunk touch distinct 16-byte bank groups of a 128- or 256-byte
// bank line, so a ds_read_b128 of a fragment is conflict-free.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return ((r >> 1) ^ (r >> 2)) & 3u; }

// Scheduling pattern of one sub-step: NM times one MFMA followed by up to V VALU instructions, and
// L direct loads, one after each of MFMAs 0, NM/4, NM/2 ...: issuing a step's loads back to back
// stalls the wave (the memory pipeline takes them one at a time) while no MFMA is queued.
template <int V, int L = 0, int NM = 16>
__device__ __forceinline__ void mfma_valu_pattern() {
#pragma unroll
  for (int q = 0; q < NM; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if (q % (NM / 4) == 0 && q / (NM / 4) < L) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
  }
}

// Two E4M3 bytes spread as (b, b, c, c) -> the fp16 pair (S_b, S_b) (HI = false) or (S_c, S_c).
template <bool HI>
__device__ __forceinline__ uint32_t scale_pair_cvt(uint32_t spread) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(spread, 1.0f, HI));
}

// Four E4M3 bytes -> four fp16 pairs (S, S).
__device__ __forceinline__ uint4 scale_pairs4(uint32_t w) {
  const uint32_t lo = __builtin_amdgcn_perm(w, w, 0x01010000u);  // b0 b0 b1 b1
  const uint32_t hi = __builtin_amdgcn_perm(w, w, 0x03030202u);  // b2 b2 b3 b3
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
  return r;
}

// OUT: 0 fp32 C, 1 bf16 C, 2 NVFP4 C (quantized in the epilogue).
// HALF: 128 x 256 tiles for the last rows of a group (at most 128 of them): each wave computes all
// 128 rows against 64 of the 256 columns (its A fragments 0-3, B fragments 0-1), half the MFMAs
// and three quarters of the decode of a full tile's wave.  The loads, the LDS ring and the waits
// are those of the full tile (A rows 128-255 of the stage read clamped rows that no wave uses).
template <int OUT, bool A2D, bool B2D, bool PAIRED, bool HALF>
__global__ __attribute__((visibility("hidden"))) __launch_bounds__(kThreads, 1) void gemm_pipe_kernel(GemmKArgs p) {
  static_assert(!HALF || OUT != 2, "the quantized epilogue takes full tiles only");
  constexpr int JN = HALF ? 2 : 4;   // B fragments per wave
  constexpr int NM = 4 * JN;         // MFMAs per sub-step
  using L = PipeLayout<PAIRED>;
  constexpr int kPStage = L::kStage, kLoadsPerStage = L::kLoadsPerStage;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[L::kBytes];
  uint8_t *const st0 = smem, *const st1 = smem + kPStage;
  uint8_t *const slots = smem + L::kScales;

  const int32_t KT = static_cast<int32_t>(p.K / 128), KP = KT / 2;  // K steps, pairs of steps
  // The workgroup's tiles: the s-th is tile_at(s) (launches with fewer workgroups than tiles run
  // each workgroup over several; every workgroup keeps its XCD).
  const int32_t nwg = static_cast<int32_t>(gridDim.x);
  auto tile_at = [&](int32_t s) {
    const int32_t v = static_cast<int32_t>(blockIdx.x) + s * nwg;
    return v < p.total_tiles ? xcd_tile(v, p.total_tiles) : -1;
  };
  struct TileRef {  // (rows of A and of B are below 2^31)
    int32_t g, m0, n0, row_end;
    const uint8_t *b_data, *b_scales;
  };
  auto describe = [&](int32_t tile) {
    TileRef t;
    int32_t g = 0;
    while (g + 1 < p.groups && p.tile_begin[g + 1] <= tile) ++g;
    const int32_t local = tile - p.tile_begin[g];
    const int32_t tiles_m_g = (p.tile_begin[g + 1] - p.tile_begin[g]) / p.tiles_n;
    int32_t tm, tn;
    band_tile(local, p.tiles_n, tiles_m_g, tm, tn);
    t.g = g;
    t.row_end = static_cast<int32_t>(p.row_end[g]);
    t.b_data = p.b_data + static_cast<int64_t>(p.group_base + g) * p.b_group_data;
    t.b_scales = p.b_scales + static_cast<int64_t>(p.group_base + g) * p.b_group_scales;
    t.m0 = static_cast<int32_t>(p.row_begin[g]) + tm * BM;
    t.n0 = tn * BN;
    return t;
  };
  TileRef cur_t = describe(tile_at(0));

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t wm = wave_row0<HALF>(wave), wn = wave_col0<HALF>(wave);

  // ---- direct-load sources: 32-bit per-lane offsets (an operand is below 2 GiB) from per-step bases
  const int64_t row_bytes = p.K / 2, KB = p.K / 16;
  uint32_t srcA[4], srcB[4];
  // PAIRED scale pairs: wave w fetches rows [64 w, 64 w + 64) of A's (even steps) or B's (odd steps)
  // slot.  Otherwise [256 rows][8 B] per operand per step: waves 0-1 stage A's, waves 2-3 B's, 64
  // dwords per load.
  uint32_t srcSA, srcSB, srcS[4];
  const bool is_a = wave < 2;
  // The per-lane offsets are kept as 32-bit values under a scalar base: each use goes through an
  // opaque copy, and the lane-derived terms are formed afresh where a tile's offsets are formed, so
  // that the compiler holds neither 64-bit addresses nor the lane terms across the K loop.
  auto opaque_u32 = [](uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
  };
  // the code sources (and, not PAIRED, the scale sources) of tile t
  auto code_sources = [&](const TileRef &t) {
    const uint32_t ln = opaque_u32(lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t R = 64 * wave + 16 * i + (ln >> 2);  // tile row this lane fetches
      const uint32_t c = (ln & 3) ^ swz(R);                 // logical chunk stored at position lane & 3
      const int64_t ra = min(static_cast<int64_t>(t.m0) + R, static_cast<int64_t>(t.row_end) - 1);
      const int64_t rb = min(static_cast<int64_t>(t.n0) + R, p.N - 1);
      srcA[i] = static_cast<uint32_t>(ra * row_bytes + 16 * c);
      srcB[i] = static_cast<uint32_t>(rb * row_bytes + 16 * c);
    }
    if constexpr (!PAIRED) {
      const int64_t r0 = is_a ? t.m0 : t.n0, r_end = is_a ? static_cast<int64_t>(t.row_end) : p.N;
      const bool two_d = is_a ? A2D : B2D;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = min(r0 + 32 * (4 * (wave & 1) + i) + (ln >> 1), r_end - 1);
        srcS[i] = static_cast<uint32_t>((two_d ? (r / 16) * KB : r * KB) + 4 * (ln & 1));
      }
    }
  };
  auto pair_sources = [&](const TileRef &t) {
    const uint32_t ln = opaque_u32(lane);
    const int64_t ra = min(static_cast<int64_t>(t.m0) + 64 * wave + ln, static_cast<int64_t>(t.row_end) - 1);
    const int64_t rb = min(static_cast<int64_t>(t.n0) + 64 * wave + ln, p.N - 1);
    srcSA = static_cast<uint32_t>(A2D ? (ra / 16) * KB : ra * KB);
    srcSB = static_cast<uint32_t>(B2D ? (rb / 16) * KB : rb * KB);
  };
  code_sources(cur_t);
  if constexpr (PAIRED) pair_sources(cur_t);
  const uint32_t lds_codes = 4096 * wave;                             // + 1024 i
  const uint32_t lds_sc = (is_a ? kPSA : kPSB) + 1024 * (wave & 1);  // + 256 i (not PAIRED)
  auto issue_codes = [&](uint8_t *st, int32_t kt) {
    const uint32_t kc = static_cast<uint32_t>(kt < KT ? kt : KT - 1);
    const uint8_t *ga = p.a_data + kc * 64u, *gb = cur_t.b_data + kc * 64u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_load16(ga + srcA[i], st + kPA + lds_codes + 1024 * i);
      lds_load16(gb + srcB[i], st + kPB + lds_codes + 1024 * i);
    }
    if constexpr (!PAIRED) {
      const uint8_t *gs = (is_a ? p.a_scales : cur_t.b_scales) + kc * 8u;
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_load4(gs + srcS[i], st + lds_sc + 256 * i);
    }
  };
  // piece i of a K step's loads: A's and B's code rows 16 i .. 16 i + 15 of each wave's 64 (and, not
  // PAIRED, the i-th scale load), step kc of the tile whose B codes / B scales start at gb / gsb
  auto issue_piece = [&](uint8_t *st, const uint8_t *gb, const uint8_t *gsb, uint32_t kc, int i) {
    lds_load16(p.a_data + kc * 64u + opaque_u32(srcA[i]), st + kPA + lds_codes + 1024 * i);
    lds_load16(gb + kc * 64u + opaque_u32(srcB[i]), st + kPB + lds_codes + 1024 * i);
    if constexpr (!PAIRED)
      lds_load4((is_a ? p.a_scales : gsb) + kc * 8u + opaque_u32(srcS[i]), st + lds_sc + 256 * i);
  };
  // PAIRED, half 0: A's scales of pair pc, half 1: B's (of the tile whose B scales start at gsb)
  auto issue_pair = [&](uint8_t *slot, const uint8_t *gsb, uint32_t pc, int half) {
    if (half == 0) lds_load16(p.a_scales + pc * 16u + opaque_u32(srcSA), slot + 1024 * wave);
    else lds_load16(gsb + pc * 16u + opaque_u32(srcSB), slot + 4096 + 1024 * wave);
  };
  // the prologue's pairs 0 and 1 (a pair past K re-fetches the last pair)
  auto issue_scales = [&](uint8_t *slot, int32_t pp, int half) {
    issue_pair(slot, cur_t.b_scales, static_cast<uint32_t>(pp < KP ? pp : KP - 1), half);
  };
  // Scale pairs are numbered on across the workgroup's tiles (pair P of its s-th tile is pair
  // s KP + P), so the ring of slots runs on from tile to tile; pair_base = (s KP) mod 3.
  // (32-bit: a wave-uniform remainder by 3 is a few scalar instructions, against ~25 in 64 bits)
  uint32_t pair_base = 0;
  auto slot_of = [&](int32_t pp) { return slots + kPSlot * ((pair_base + static_cast<uint32_t>(pp)) % 3u); };

  // ---- fragment reads: lane half h takes codes [64 h, 64 h + 64) of the step, chunk q of its half
  const uint32_t rdA = (wm + l32) * 64, rdB = (wn + l32) * 64;
  const uint32_t pos0 = 16 * ((2 * h) ^ swz(l32)), pos1 = 16 * ((2 * h + 1) ^ swz(l32));
  const uint32_t rsA = PAIRED ? (wm + l32) * 16 + 4 * h : kPSA + (wm + l32) * 8 + 4 * h;
  const uint32_t rsB = PAIRED ? 4096 + (wn + l32) * 16 + 4 * h : kPSB + (wn + l32) * 8 + 4 * h;
  auto read_chunk = [&](const uint8_t *st, uint32_t pos, uint4 (&ca)[4], uint4 (&cb)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      ca[f] = *reinterpret_cast<const uint4 *>(st + kPA + rdA + 2048 * f + pos);
      if (f < JN) cb[f] = *reinterpret_cast<const uint4 *>(st + kPB + rdB + 2048 * f + pos);
    }
  };
  // the scale words of step kt (blocks 4 h .. 4 h + 3): out of its pair's slot, or its stage
  auto read_scales = [&](const uint8_t *src, int32_t kt, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
    const uint32_t par = PAIRED ? 8 * static_cast<uint32_t>(kt & 1) : 0u;
    constexpr uint32_t kFrag = PAIRED ? 512 : 256;  // 32 rows
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sa[f] = *reinterpret_cast<const uint32_t *>(src + rsA + par + kFrag * f);
      if (f < JN) sb[f] = *reinterpret_cast<const uint32_t *>(src + rsB + par + kFrag * f);
    }
  };

  floatx16 acc[4][4];  // [B fragment j][A fragment i] (j < JN)
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  // ---- prologue: steps 0 and 1 and scale pairs 0 and 1 in flight, step 0's first chunk read and
  // its sub-step 0 decoded
  if constexpr (PAIRED) {
    issue_scales(slots, 0, 0);
    issue_scales(slots, 0, 1);
  }
  issue_codes(st0, 0);
  if constexpr (PAIRED) {
    issue_scales(slots + kPSlot, 1, 0);
    issue_scales(slots + kPSlot, 1, 1);
  }
  issue_codes(st1, 1);
  wait_vmcnt<PAIRED ? 10 : kLoadsPerStage>();  // step 1 (and pair 1) may still be in flight
  lds_barrier();
  uint4 ca0[4], cb0[4], ca1[4], cb1[4];  // chunk 0 / chunk 1 codes of the current step
  uint4 psa[4], psb[4];                   // fp16 scale pairs of the current step (blocks 4h..4h+3)
  half8 afc[4], bfc[4];                   // the current sub-step's decoded fragments
  // a tile's step 0 (in stage st, its scale pair 0 in slot sc, both complete): its first chunk and
  // scales read and its sub-step 0 decoded
  auto start_tile = [&](const uint8_t *st, const uint8_t *sc) {
    uint32_t rsa[4], rsb[4];
    read_chunk(st, pos0, ca0, cb0);
    read_scales(PAIRED ? sc : st, 0, rsa, rsb);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      psa[f] = scale_pairs4(rsa[f]);
      if (f < JN) psb[f] = scale_pairs4(rsb[f]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      afc[f] = decode8(ca0[f].x, psa[f].x);
      if (f < JN) bfc[f] = decode8(cb0[f].x, psb[f].x);
    }
  };
  start_tile(st0, slots);

  // one K step out of stage cur: the 8 sub-steps of 16 codes, 16 MFMAs each.  sc_nxt holds the next
  // step's scale pair, sc_tgt receives half of a later pair (distinct slots).
  // The next step's scale words (read after the barrier in sub-step 4) become fp16 pairs in three
  // parts, each written over components of psa / psb that this step no longer reads: the decodes of
  // sub-steps 6 and 7 (issued in iterations 5 and 6) read component 3 only, so components 0 and 1
  // are converted in iteration 5, component 2 in iteration 6 and component 3 in iteration 7, where
  // the next step's sub-step 0 is decoded.
  // Steps and pairs past the tile's K are the next tile's first ones (nxt_t, where it has one: its
  // sources replace this tile's from the step that first loads for it on, step KT - 4 for the scale
  // pairs and KT - 2 for the codes), else a re-fetch of the last step / pair into a stage or slot
  // that is never consumed.
  TileRef nxt_t = cur_t;
  bool has_next = false;
  // (tail: one of the tile's last four steps, the only ones that may load past its K; the others
  // are a loop of their own that holds no state of the next tile)
  auto step = [&](uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt, uint8_t *__restrict__ tgt,
                  const uint8_t *__restrict__ sc_nxt, uint8_t *__restrict__ sc_tgt, int32_t kt, bool tail) {
    // what this step loads: codes of step kt + 2 and (PAIRED) half kt & 1 of pair (kt + 4) / 2
    const int32_t jc = kt + 2, jp = (kt + 4) >> 1;
    const bool c_next = tail && has_next && jc >= KT, p_next = tail && has_next && jp >= KP;
    const uint32_t kc = static_cast<uint32_t>(!tail || jc < KT ? jc : (c_next ? jc - KT : KT - 1));
    const uint32_t pc = static_cast<uint32_t>(!tail || jp < KP ? jp : (p_next ? jp - KP : KP - 1));
    const uint8_t *const gb = c_next ? nxt_t.b_data : cur_t.b_data;
    const uint8_t *const gsb = (PAIRED ? p_next : c_next) ? nxt_t.b_scales : cur_t.b_scales;
    if (tail && has_next && kt == KT - 2) code_sources(nxt_t);
    if constexpr (PAIRED)
      if (tail && has_next && kt == KT - 4) pair_sources(nxt_t);
    read_chunk(cur, pos1, ca1, cb1);
    // the reads go out now, three sub-steps before their first use (left to itself the compiler
    // sinks each read next to its use and waits for it there)
    __builtin_amdgcn_sched_barrier(0);
    uint32_t nsa[4], nsb[4];  // next step's raw scale bytes
    uint32_t hia[4], hib[4];  // their bytes 2 and 3 spread into pairs
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      half8 afn[4], bfn[4];
      if (m < 7) {
        const int mn = m + 1;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint32_t da = mn < 4 ? pick(ca0[f], mn) : pick(ca1[f], mn - 4);
          afn[f] = decode8(da, pick(psa[f], mn >> 1));
          if (f < JN) {
            const uint32_t db = mn < 4 ? pick(cb0[f], mn) : pick(cb1[f], mn - 4);
            bfn[f] = decode8(db, pick(psb[f], mn >> 1));
          }
        }
      }
      if (m == 5) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint32_t loa = __builtin_amdgcn_perm(nsa[f], nsa[f], 0x01010000u);  // b0 b0 b1 b1
          psa[f].x = scale_pair_cvt<false>(loa);
          psa[f].y = scale_pair_cvt<true>(loa);
          if (f < JN) {
            const uint32_t lob = __builtin_amdgcn_perm(nsb[f], nsb[f], 0x01010000u);
            psb[f].x = scale_pair_cvt<false>(lob);
            psb[f].y = scale_pair_cvt<true>(lob);
          }
        }
      } else if (m == 6) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          hia[f] = __builtin_amdgcn_perm(nsa[f], nsa[f], 0x03030202u);  // b2 b2 b3 b3
          psa[f].z = scale_pair_cvt<false>(hia[f]);
          if (f < JN) {
            hib[f] = __builtin_amdgcn_perm(nsb[f], nsb[f], 0x03030202u);
            psb[f].z = scale_pair_cvt<false>(hib[f]);
          }
        }
      } else if (m == 7) {
        // this step's chunk 0 is dead: ca0 / cb0 hold the next step's chunk 0 (read after the
        // barrier of sub-step 4)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          psa[f].w = scale_pair_cvt<true>(hia[f]);
          afn[f] = decode8(ca0[f].x, psa[f].x);
          if (f < JN) {
            psb[f].w = scale_pair_cvt<true>(hib[f]);
            bfn[f] = decode8(cb0[f].x, psb[f].x);
          }
        }
      }
      // the loads of step kt + 2 (into the stage of step kt - 1, free since the barrier of step
      // kt - 1), a quarter per sub-step 0-3: all are issued before this step's barrier
      if (m < 4) {
        issue_piece(tgt, gb, gsb, kc, m);
        if constexpr (PAIRED)
          if (m == 0) issue_pair(sc_tgt, gsb, pc, kt & 1);
      }
#pragma unroll
      for (int j = 0; j < JN; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfc[j], afc[i], acc[j][i], 0, 0, 0);
      // one MFMA, then the VALU work of the sub-step spread evenly (four decode instructions, five or
      // six where scale conversions join them; HALF: six decode instructions per MFMA, eight or nine
      // with the conversions): the matrix pipe is never left behind a long run of VALU work (a wave
      // issues in order)
      constexpr int VD = HALF ? 6 : 4;
      if (m == 5)
        mfma_valu_pattern<HALF ? 9 : 6, 0, NM>();
      else if (m >= 6)
        mfma_valu_pattern<HALF ? 8 : 5, 0, NM>();
      else if (m == 0)
        mfma_valu_pattern<VD, 3, NM>();
      else if (m < 4)
        mfma_valu_pattern<VD, PAIRED ? 2 : 3, NM>();
      else
        mfma_valu_pattern<VD, 0, NM>();
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        afc[f] = afn[f];
        if (f < JN) bfc[f] = bfn[f];
      }
      if (m == 4) {
        // every wave holds this step's codes in registers (chunk 1 since sub-step 3's decode), and
        // this lane's loads for step kt + 1 have landed: after the barrier the next stage is complete
        // and this one may be refilled.  (Fenced on both sides: MFMAs and decodes touch no memory, so
        // the scheduler would otherwise move the barrier and its waits far up the step.)
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kLoadsPerStage>();
        wait_lgkmcnt0();
        lds_barrier();
        read_chunk(nxt, pos0, ca0, cb0);
        read_scales(PAIRED ? sc_nxt : nxt, kt + 1, nsa, nsb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  uint8_t *cur = st0, *nxt = st1, *tgt = smem + 2 * kPStage;
  const float ts_a = *p.a_ts;
  for (int32_t s = 0;; ++s) {
    // (bf16 C, or fp32 C with paired scale loads (the unpaired fp32 kernel would spill), and at
    // least four K steps: the tile's C is staged in the one free stage, fp32 one 64-column half at a
    // time, and the next tile's first scale pair is fetched from step KT - 4 on)
    auto run_steps = [&](int32_t k0, int32_t k1, bool tail) __attribute__((always_inline)) {
      for (int32_t kt = k0; kt < k1; ++kt) {
        if constexpr (PAIRED) step(cur, nxt, tgt, slot_of((kt + 1) >> 1), slot_of((kt + 4) >> 1), kt, tail);
        else step(cur, nxt, tgt, nullptr, nullptr, kt, tail);
        uint8_t *const done = cur;
        cur = nxt;
        nxt = tgt;
        tgt = done;
      }
    };
    const int32_t k_tail = KT > 4 ? KT - 4 : 0;
    run_steps(0, k_tail, false);
    const int32_t next_tile = (OUT == 1 || (OUT == 0 && PAIRED)) && KT >= 4 ? tile_at(s + 1) : -1;
    has_next = next_tile >= 0;
    if (has_next) nxt_t = describe(next_tile);
    run_steps(k_tail, KT, true);

    // ---- epilogue: C = acc * ts_a * ts_b (one multiply where ts_a * ts_b is a normal number)
    const float ts_b = p.b_ts[p.group_base + cur_t.g];
    if constexpr (OUT == 2) {
      float amax = store_q_tile(acc, smem, p.q_data, p.q_scales, p.N, cur_t.m0, cur_t.n0, cur_t.row_end, ts_a, ts_b,
                                *p.q_ts, wave, lane);
      if (p.amax != nullptr) {
        // non-negative floats order like their bit patterns: one atomic max per wave
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) atomicMax(reinterpret_cast<unsigned int *>(p.amax), __float_as_uint(amax));
      }
    } else if (!has_next) {
      store_c_tile<OUT == 1, HALF>(acc, smem, p.c, p.ldc, cur_t.m0, cur_t.n0, cur_t.row_end, p.N, ts_a, ts_b,
                                   p.vec_store != 0, wave, lane);
    } else {
      // staged in tgt, the stage of the tile's last step: read by no wave since that step's barrier
      // and the target of the next tile's first loads, so every wave's read-back completes before
      // the barrier after it; the next tile's loads in flight are not waited for
      store_c_tile<OUT == 1, HALF, true>(acc, tgt, p.c, p.ldc, cur_t.m0, cur_t.n0, cur_t.row_end, p.N, ts_a,
                                         ts_b, p.vec_store != 0, wave, lane, false);
      wait_lgkmcnt0();
      lds_barrier();
    }
    if (!has_next) break;
    // the next tile: its steps 0 and 1 and scale pairs 0 and 1 are loaded (step 0 and pair 0
    // complete since the last step's barrier), so its start is read again from LDS (cheaper than
    // holding the last step's reads of it in registers through the epilogue)
    cur_t = nxt_t;
    pair_base = (pair_base + static_cast<uint32_t>(KP)) % 3u;
    start_tile(cur, slot_of(0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;
  }
}


// Launch of one variant: OUT 0 fp32 C, 1 bf16 C, 2 NVFP4 C; the pipelined kernel for whole K steps
// (full), with block scales two steps per load (paired), else the bounds-checked kernel.  grid:
// workgroups (p.total_tiles, or fewer for the pipelined kernel with bf16 C and at least four K
// steps, whose workgroups then run several tiles each).
template <int OUT, bool A2D, bool B2D>
hipError_t launch_variant(const GemmKArgs &p, int32_t grid, bool full, bool paired, bool half, hipStream_t stream) {
  if (half) {
    // 128 x 256 tiles: the paired pipelined kernel with fp32 or bf16 C only
    if constexpr (OUT == 2) return hipErrorInvalidValue;
    else if (!paired) return hipErrorInvalidValue;
    else hipLaunchKernelGGL((gemm_pipe_kernel<OUT, A2D, B2D, true, true>), dim3(grid), dim3(kThreads), 0, stream, p);
  } else if (paired)
    hipLaunchKernelGGL((gemm_pipe_kernel<OUT, A2D, B2D, true, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  else if constexpr (OUT == 2)
    return hipErrorInvalidValue;  // the quantized epilogue exists in the paired kernel only
  else if (full)
    hipLaunchKernelGGL((gemm_pipe_kernel<OUT, A2D, B2D, false, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_kernel<OUT == 1, A2D, B2D, false>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

#define NVFP4_GEMM_VARIANTS(X) \
  X(0, false, false) X(0, false, true) X(0, true, false) X(0, true, true) \
  X(1, false, false) X(1, false, true) X(1, true, false) X(1, true, true) \
  X(2, false, false) X(2, false, true) X(2, true, false) X(2, true, true)

}  // namespace gemm
}  // namespace nvfp4
