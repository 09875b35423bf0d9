// probe_designs.hip -- measurement probe for the choice of GEMM design (built as libnvfp4_probe.so;
// not part of the library's ABI).
//
// NVFP4 scales every 16 consecutive K elements with their own E4M3 scale.  The two ways to put the
// block-scaled product on CDNA4 matrix cores are run here on the same inner step: one wave computes
// a 128 x 128 tile (4 x 4 tiles of 32 x 32, the library's wave tile) over one 16-element K block,
// `reps` times, from operands held in registers (so only the inner step is timed, no memory):
//   design 0 (the library's): each code decoded exactly to fp16 with its scale folded in
//            (v_cvt_scalef32_pk_f16_fp4, v_pk_mul_f16), then v_mfma_f32_32x32x16_f16 accumulating
//            straight into the tile: 16 MFMAs and 64 VALU instructions per block.
//   design 1: the codes as they are, fp4 operands of v_mfma_scale_f32_32x32x64_f8f6f4 (64 K per
//            instruction, so the block fills a quarter of it and the rest is zero; its scale operands
//            are E8M0, one per 32 K, which cannot carry an E4M3 scale), into a fresh accumulator per
//            32 x 32 tile, then rescaled into the tile: acc += partial * (S_a[row] * S_b[col]),
//            two VALU instructions per output element: 16 MFMAs and 512 VALU instructions per block.
// A third variant runs design 0's MFMAs alone, on operands decoded once.
// All write the wave's tile of C = sum_k (q_a S_a)(q_b S_b) (reps = 1: one block) for the test
// that checks them against the oracle.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef int int8v __attribute__((ext_vector_type(8)));

// E4M3 byte -> its value (exact in fp32; the hardware fp8 decode).
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(b, 1.0f, false);
  return v[0];
}

// 8 codes (code n at bits 4n) times the fp16 pair (S, S) -> 8 exact fp16 values.
__device__ __forceinline__ half8 decode8(uint32_t w, half2v s2) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The probe repeats one block; in a GEMM every block brings new codes and scales.  An empty asm
// with a read-write register constraint makes a value opaque (no instruction is emitted), so the
// compiler cannot hoist the per-block work out of the repetition loop.
template <class T>
__device__ __forceinline__ void opaque(T &v) {
  asm volatile("" : "+v"(v));
}

struct ProbeArgs {
  const uint8_t *a_codes, *a_scales;  // A [128][16 codes]: 8 bytes per row; one scale byte per row
  const uint8_t *b_codes, *b_scales;  // B [128][16 codes], one scale byte per row
  float *c;                           // [128][128] (written by wave 0 of workgroup 0)
  int reps;
};

// Output element r of a 32 x 32 MFMA tile held by lane l: row 8 (r >> 2) + 4 (l >> 5) + (r & 3),
// column l & 31.
template <int TM = 4, int TN = 4>
__device__ __forceinline__ void write_tile(const floatx16 (&acc)[4][4], float *c, uint32_t lane) {
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t row = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), col = 32 * j + (lane & 31);
        c[row * 128 + col] = acc[i][j][r];
      }
}

// Design 0 on a wave tile of TM x TN MFMA tiles (the library's is 4 x 4), NT threads per workgroup
// (256: one wave per SIMD; 512: two, which a 2 x 4 tile's 128 accumulators allow).
// DECODE: 1 = each use decodes its operands (the library's K loop), 0 = the MFMAs alone on operands
// decoded once, 2 = the MFMAs on operands decoded once plus the same decode work on other registers
// (independent of the MFMAs: whether a wave's VALU work overlaps its own MFMAs at all), 3 = as 2 with
// conversions only (eight independent v_cvt per 8 codes instead of four conversions and four
// multiplies that depend on them).
template <int TM, int TN, int DECODE, int NT>
__global__ __launch_bounds__(NT, 1) void probe_fp16_decode(ProbeArgs p) {
  const uint32_t lane = threadIdx.x & 63u, l32 = lane & 31u, h = lane >> 5;
  // this lane's codes of K 8h .. 8h + 7 (one dword) and its row's scale, per A and B fragment
  uint32_t ca[TM], cb[TN];
  half2v sa[TM], sb[TN];
#pragma unroll
  for (int f = 0; f < TM; ++f) {
    const uint32_t row = 32 * f + l32;
    ca[f] = reinterpret_cast<const uint32_t *>(p.a_codes + row * 8)[h];
    const _Float16 s_a = static_cast<_Float16>(e4m3_value(p.a_scales[row]));
    sa[f] = half2v{s_a, s_a};
  }
#pragma unroll
  for (int f = 0; f < TN; ++f) {
    const uint32_t row = 32 * f + l32;
    cb[f] = reinterpret_cast<const uint32_t *>(p.b_codes + row * 8)[h];
    const _Float16 s_b = static_cast<_Float16>(e4m3_value(p.b_scales[row]));
    sb[f] = half2v{s_b, s_b};
  }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx16{};
  half8 af[TM], bf[TN];
#pragma unroll
  for (int f = 0; f < TM; ++f) af[f] = decode8(ca[f], sa[f]);
#pragma unroll
  for (int f = 0; f < TN; ++f) bf[f] = decode8(cb[f], sb[f]);
  for (int rep = 0; rep < p.reps; ++rep) {
    half8 ta[TM], tb[TN];  // DECODE == 2, 3: decoded values that no MFMA reads
    if constexpr (DECODE == 3) {
      auto cvt8 = [](uint32_t w) {
        const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
        const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
        const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
        const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
        const half2v q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0);
        const half2v q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1);
        const half2v q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2);
        const half2v q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3);
        half8 r0 = half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        half8 r1 = half8{q0[0], q0[1], q1[0], q1[1], q2[0], q2[1], q3[0], q3[1]};
        opaque(r1);
        return r0;
      };
#pragma unroll
      for (int f = 0; f < TM; ++f) ta[f] = cvt8(ca[f] ^ static_cast<uint32_t>(rep));
#pragma unroll
      for (int f = 0; f < TN; ++f) tb[f] = cvt8(cb[f] ^ static_cast<uint32_t>(rep));
    } else if constexpr (DECODE == 2) {
      // codes that change with the repetition (one v_xor), so the decode cannot be hoisted
#pragma unroll
      for (int f = 0; f < TM; ++f) ta[f] = decode8(ca[f] ^ static_cast<uint32_t>(rep), sa[f]);
#pragma unroll
      for (int f = 0; f < TN; ++f) tb[f] = decode8(cb[f] ^ static_cast<uint32_t>(rep), sb[f]);
    } else if constexpr (DECODE == 1) {
      // the decode of every use, as in the library's K loop (the codes differ from block to block)
#pragma unroll
      for (int f = 0; f < TM; ++f) {
        opaque(ca[f]);
        af[f] = decode8(ca[f], sa[f]);
      }
#pragma unroll
      for (int f = 0; f < TN; ++f) {
        opaque(cb[f]);
        bf[f] = decode8(cb[f], sb[f]);
      }
    } else {
      // the MFMAs alone: operands decoded once, only made opaque
#pragma unroll
      for (int f = 0; f < TM; ++f) opaque(af[f]);
#pragma unroll
      for (int f = 0; f < TN; ++f) opaque(bf[f]);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    if constexpr (DECODE >= 2) {
      // one MFMA, then its share of the decode instructions, throughout
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 9 * (TM + TN) / (TM * TN), 0);
      }
#pragma unroll
      for (int f = 0; f < TM; ++f) opaque(ta[f]);
#pragma unroll
      for (int f = 0; f < TN; ++f) opaque(tb[f]);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) write_tile<TM, TN>(acc, p.c, lane);
}

// Design 0 software-pipelined, as the library's K loop: the decode of repetition r + 1 (codes that
// change with r, one v_xor) is interleaved with the MFMAs of repetition r, one MFMA then its share
// of the decode instructions (4 x 4 tile, one wave per SIMD).
__global__ __launch_bounds__(256, 1) void probe_fp16_pipelined(ProbeArgs p) {
  const uint32_t lane = threadIdx.x & 63u, l32 = lane & 31u, h = lane >> 5;
  uint32_t ca[4], cb[4];
  half2v sa[4], sb[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint32_t row = 32 * f + l32;
    ca[f] = reinterpret_cast<const uint32_t *>(p.a_codes + row * 8)[h];
    cb[f] = reinterpret_cast<const uint32_t *>(p.b_codes + row * 8)[h];
    const _Float16 s_a = static_cast<_Float16>(e4m3_value(p.a_scales[row]));
    const _Float16 s_b = static_cast<_Float16>(e4m3_value(p.b_scales[row]));
    sa[f] = half2v{s_a, s_a};
    sb[f] = half2v{s_b, s_b};
  }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
  half8 af[4], bf[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    af[f] = decode8(ca[f], sa[f]);
    bf[f] = decode8(cb[f], sb[f]);
  }
  half8 an[4], bn[4];
  // MFMAs on (ac, bc) interleaved with the decode of the next block into (ad, bd)
  auto block = [&](const half8 (&ac)[4], const half8 (&bc)[4], half8 (&ad)[4], half8 (&bd)[4]) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint32_t da = ca[f], db = cb[f];
      opaque(da);
      opaque(db);
      ad[f] = decode8(da, sa[f]);
      bd[f] = decode8(db, sb[f]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ac[i], bc[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };
  for (int rep = 0; rep < p.reps; rep += 2) {  // (reps even)
    block(af, bf, an, bn);
    block(an, bn, af, bf);
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) write_tile(acc, p.c, lane);
}

__global__ __launch_bounds__(256, 1) void probe_fp4_rescale(ProbeArgs p) {
  const uint32_t lane = threadIdx.x & 63u, l32 = lane & 31u, h = lane >> 5;
  // fp4 operands: lane l holds K 32 (l >> 5) .. +31 of row l & 31; the block is K 0..15, the rest
  // zero
  int8v a[4], b[4];
  float sar[4][16], sbc[4];  // S_a of the lane's 16 output rows per A fragment; S_b of its column
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint32_t row = 32 * f + l32;
    const uint2 va = h == 0 ? *reinterpret_cast<const uint2 *>(p.a_codes + row * 8) : make_uint2(0, 0);
    const uint2 vb = h == 0 ? *reinterpret_cast<const uint2 *>(p.b_codes + row * 8) : make_uint2(0, 0);
    a[f] = int8v{static_cast<int>(va.x), static_cast<int>(va.y), 0, 0, 0, 0, 0, 0};
    b[f] = int8v{static_cast<int>(vb.x), static_cast<int>(vb.y), 0, 0, 0, 0, 0, 0};
    sbc[f] = e4m3_value(p.b_scales[row]);
#pragma unroll
    for (int r = 0; r < 16; ++r) sar[f][r] = e4m3_value(p.a_scales[32 * f + 8 * (r >> 2) + 4 * h + (r & 3)]);
  }
  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx16{};
  for (int rep = 0; rep < p.reps; ++rep) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      opaque(a[f]);
      opaque(b[f]);
      opaque(sbc[f]);
#pragma unroll
      for (int r = 0; r < 16; ++r) opaque(sar[f][r]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // 127 = E8M0 1.0: the partial sum of q_a q_b over the block, exact
        const floatx16 part = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], floatx16{}, 4, 4, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(part[r], sar[i][r] * sbc[j], acc[i][j][r]);
      }
  }
  if (blockIdx.x == 0 && threadIdx.x < 64) write_tile(acc, p.c, lane);
}

}  // namespace

// design: 0 = fp16 decode + f16 MFMA, 1 = fp4 MFMA + per-block rescale, 2 = the f16 MFMAs of
// design 0 alone (operands decoded once: the cost of the decode is the difference); on a 2 x 4 wave
// tile (64 x 128): 3 = design 0 with two waves per SIMD, 4 = design 0 with one, 5 = design 2 with
// two; 6 = design 2 plus design 0's decode work on registers the MFMAs do not read (4 x 4 tile, one
// wave per SIMD); 7 = design 0 software-pipelined (4 x 4 tile, one wave per SIMD); 8 = design 6 with
// conversions only (no VALU instruction waits for another).  Designs 0-2 and 6 run workgroups of 4 waves (one per SIMD), 3-5 of 8 or 4; every
// wave runs the same step; returns 0, or the HIP error code of the launch.
extern "C" __attribute__((visibility("default"))) int nvfp4_probe_design(int design, const uint8_t *a_codes,
                                                                         const uint8_t *a_scales, const uint8_t *b_codes,
                                                                         const uint8_t *b_scales, float *c, int reps,
                                                                         int workgroups, void *stream) {
  ProbeArgs p{a_codes, a_scales, b_codes, b_scales, c, reps};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // 96 KB of LDS per workgroup (unused) keeps one workgroup per CU for the 2 x 4 tiles, so their
  // waves per SIMD are exactly 2 (512 threads) or 1 (256)
  const size_t one_per_cu = 96 * 1024;
  if (design == 0)
    hipLaunchKernelGGL((probe_fp16_decode<4, 4, 1, 256>), dim3(workgroups), dim3(256), 0, st, p);
  else if (design == 2)
    hipLaunchKernelGGL((probe_fp16_decode<4, 4, 0, 256>), dim3(workgroups), dim3(256), 0, st, p);
  else if (design == 3)
    hipLaunchKernelGGL((probe_fp16_decode<2, 4, 1, 512>), dim3(workgroups), dim3(512), one_per_cu, st, p);
  else if (design == 4)
    hipLaunchKernelGGL((probe_fp16_decode<2, 4, 1, 256>), dim3(workgroups), dim3(256), one_per_cu, st, p);
  else if (design == 5)
    hipLaunchKernelGGL((probe_fp16_decode<2, 4, 0, 512>), dim3(workgroups), dim3(512), one_per_cu, st, p);
  else if (design == 6)
    hipLaunchKernelGGL((probe_fp16_decode<4, 4, 2, 256>), dim3(workgroups), dim3(256), 0, st, p);
  else if (design == 7)
    hipLaunchKernelGGL(probe_fp16_pipelined, dim3(workgroups), dim3(256), 0, st, p);
  else if (design == 8)
    hipLaunchKernelGGL((probe_fp16_decode<4, 4, 3, 256>), dim3(workgroups), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(probe_fp4_rescale, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}
