// nvfp4_device.hpp -- device-side building blocks of the NVFP4 kernels (gfx950).
//
// Every floating-point step that decides a bit of the output is one IEEE binary32 operation, in
// the order the library's format definition lists (include/nvfp4.h).  The sources are compiled
// with -ffp-contract=off so that no multiply and add are fused unless written as fmaf, and '/' is
// the correctly rounded division sequence (v_div_scale / v_div_fmas / v_div_fixup).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

enum Mode : int { kRNE = 0, kSR = 1, kFourOverSix = 2, kSearch = 3 };

// ---- bf16 / f32 unpacking --------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- E4M3 (FN) block scale -------------------------------------------------------------------
// Round s in [0, 448] to the nearest E4M3FN value, ties to even mantissa.  Returns the byte and
// the decoded value (the rounded fp32 number itself).
__device__ __forceinline__ uint32_t e4m3_rne(float s, float &S) {
  if (s < 0.015625f) {                         // below 2^-6: E4M3 subnormals, spacing 2^-9
    float m = __builtin_rintf(s * 512.0f);     // exact scaling, then nearest-even integer 0..8
    S = m * 0.001953125f;
    return static_cast<uint32_t>(m);           // m == 8 encodes 2^-6, the smallest normal
  }
  uint32_t b = __float_as_uint(s);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;  // keep 3 mantissa bits, RNE
  S = __uint_as_float(r);
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);  // exponent rebias 127 -> 7
}

// Block scale for block maximum ab and grid target T (6, or 4 under Four-over-Six).
__device__ __forceinline__ uint32_t block_scale(float ab, float T, float ts, float &S) {
  if (ts == 0.0f) {
    S = 0.0f;
    return 0u;
  }
  float q = ab / T;
  float s = q / ts;
  s = fminf(s, 448.0f);
  return e4m3_rne(s, S);
}

// Per-block encode factor e = RN(1 / RN(S * ts)); 0 for a zero scale (every code is then a signed
// zero).  e is +inf only when S * ts underflows, a degenerate case handled element-wise.
__device__ __forceinline__ float encode_factor(float S, float ts) {
  if (S == 0.0f) return 0.0f;
  float d = S * ts;
  return 1.0f / d;
}

// ---- E2M1 element rounding ---------------------------------------------------------------------
// v >= 0 (not NaN): index 0..7 of the nearest value of {0,0.5,1,1.5,2,3,4,6}, ties to the even
// index, saturating at 6.  Below 1 the grid has spacing 0.5: adding 2^22 (whose ulp is 0.5) rounds
// to it nearest-even.  From 1 up the grid is the floats with one mantissa bit: round the fp32
// mantissa to one bit (nearest-even) and read exponent and bit as the index.
__device__ __forceinline__ uint32_t e2m1_rne_index(float v) {
  float vc = fminf(v, 6.0f);
  uint32_t small = __float_as_uint(vc + 4194304.0f) & 7u;
  uint32_t b = __float_as_uint(vc);
  uint32_t big = ((b + 0x11FFFFFu + ((b >> 22) & 1u)) >> 22) & 15u;
  return vc < 1.0f ? small : big;
}

// ---- nearest-even block encode (shared by the quantize passes and the GEMM's quantized epilogue) ------
__device__ __forceinline__ uint32_t sign_code(float y) { return (__float_as_uint(y) >> 28) & 8u; }

// e == +inf (S * ts underflowed): nonzero elements saturate to 6, zeros stay zero.
__device__ __forceinline__ uint32_t code_degenerate(float y) {
  return (y == 0.0f ? 0u : 7u) | sign_code(y);
}

// Nearest-even codes of 8 values times e, packed (code n at bits 4n).  The hardware conversion
// (scale 1.0) rounds to nearest-even and saturates at 6.
__device__ __forceinline__ uint32_t pack8_rne(const float *y, float e) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0] * e, y[1] * e, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2] * e, y[3] * e, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4] * e, y[5] * e, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6] * e, y[7] * e, 1.0f, 3);
  return w;
}

__device__ __forceinline__ float block_absmax(const float (&y)[16]) {
  float ab = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) ab = fmaxf(ab, fabsf(y[t]));
  return ab;
}

// One 1D block, nearest-even: scale byte and the two packed code words.
__device__ __forceinline__ void encode_block_rne(const float (&y)[16], float ab, float ts, uint32_t &sbyte,
                                                 uint32_t &w0, uint32_t &w1) {
  float S;
  sbyte = block_scale(ab, 6.0f, ts, S);
  const float e = encode_factor(S, ts);
  if (__builtin_isinf(e)) {
    w0 = 0u;
    w1 = 0u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      w0 |= code_degenerate(y[t]) << (4 * t);
      w1 |= code_degenerate(y[8 + t]) << (4 * t);
    }
  } else {
    w0 = pack8_rne(y, e);
    w1 = pack8_rne(y + 8, e);
  }
}

// ---- Philox4x32-10 -------------------------------------------------------------------------------
// Counter-based generator of Salmon et al. (SC 2011): ten rounds of two 32x32->64 multiplies with
// the multipliers 0xD2511F53 / 0xCD9E8D57, key bumped by the Weyl increments 0x9E3779B9 /
// 0xBB67AE85 between rounds.
struct u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // full 64-bit products: one v_mad_u64_u32 each gives both halves
    const uint64_t p0 = static_cast<uint64_t>(c0) * 0xD2511F53u;
    const uint64_t p1 = static_cast<uint64_t>(c2) * 0xCD9E8D57u;
    // three-way XORs as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(static_cast<uint32_t>(p0 >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = static_cast<uint32_t>(p1);
    c2 = n2;
    c3 = static_cast<uint32_t>(p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// ---- 16-point random Hadamard transform (in registers) -------------------------------------------
// u <- (1/4) H16 D u: signs from the low 16 bits of sign_word, then the radix-2 butterfly with
// strides 1, 2, 4, 8 (a + b to the lower, a - b to the upper slot), then the exact multiply by 1/4.
__device__ __forceinline__ void rht16(float (&u)[16], uint32_t sign_word) {
#pragma unroll
  for (int t = 0; t < 16; ++t) u[t] = __uint_as_float(__float_as_uint(u[t]) ^ (((sign_word >> t) & 1u) << 31));
#pragma unroll
  for (int h = 1; h < 16; h *= 2) {
#pragma unroll
    for (int i = 0; i < 16; i += 2 * h) {
#pragma unroll
      for (int m = i; m < i + h; ++m) {
        float a = u[m], b = u[m + h];
        u[m] = a + b;
        u[m + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) u[t] = u[t] * 0.25f;
}

// ---- fast division by a run-time invariant 32-bit divisor ----------------------------------------
// Granlund & Montgomery, "Division by invariant integers using multiplication" (PLDI 1994),
// the unsigned round-up method: q = (t + ((n - t) >> s1)) >> s2 with t = mulhi(m, n).
struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0, 0, 0};
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.m = static_cast<uint32_t>(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
  uint32_t t = __umulhi(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// ---- wave / workgroup reductions ------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}

}  // namespace nvfp4
