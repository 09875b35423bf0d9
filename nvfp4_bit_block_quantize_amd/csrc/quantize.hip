// quantize.hip -- NVFP4 quantize kernels for gfx950 (HBM-bound).
//
// Two passes per tensor, both on the caller's stream:
//   pass 1  tensor amax: every workgroup writes the largest |y| it saw to workspace[blockIdx.x]
//           (plain tensors: amax_kernel; with the Hadamard transform the maximum is taken over the
//           transformed values: row1d_kernel compiled with PASS1 = true, col_amax_kernel);
//   pass 2  every workgroup reduces the partial maxima itself (no atomics, no zeroed memory),
//           derives ts = amax / 2688, and encodes its blocks: block amax -> E4M3 scale -> E2M1
//           codes (nearest-even, stochastic or Four-over-Six) -> packed nibbles.
// Pass-2 grids are persistent (a few workgroups per CU, grid-stride over the work) so that the
// partial reduction is paid a few times per CU, and each lane issues the loads of its
// next block before it encodes the current one.
//
// Nearest-even encoding uses v_cvt_scalef32_pk_fp4_f32 with scale 1.0: two fp32 values -> two
// E2M1 codes (sign copied, ties to even, saturating at 6) packed into a chosen byte.  On MI355X
// this instruction agrees with the format's rounding rule on every one of the 2^32 fp32 inputs
// except NaN (checked exhaustively), so v = y * e is fed to it directly.
//
// Layouts:
//   row1d_kernel    ROW mode, 1D blocks: one lane per 16-element block (32 B of bf16 in, 8 B out).
//   row2d_kernel    ROW mode, 16x16 tiles: a lane holds 16 rows x 8 columns; a lane pair is a tile.
//   col_kernel      COLWISE: a lane holds 16 tokens x CPL columns (8, or 4 for stochastic
//                   rounding), i.e. one block of each of CPL rows of x^T; a 256-lane workgroup
//                   covers 256 tokens x 16 CPL columns and transposes its packed output through LDS
//                   so that every row segment leaves as 128 contiguous bytes.
//   col_amax_kernel COLWISE pass 1 with the transform: a wave reads 16 rows x 1 KiB strips.
#include <type_traits>

#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr uint32_t kThreads = 256;
constexpr uint32_t kPass1Parts = 1024; // pass-1 workgroups at most (<= kMaxParts): the partial maxima
                                       // every pass-2 wave reduces
constexpr uint32_t kAmaxThreads = 1024; // amax_kernel workgroup: one per CU, 16 waves
constexpr uint32_t kAmaxParts = 256;
constexpr uint32_t kPass2Grid = 2048;  // persistent pass-2 workgroups (8 per CU)
// row2d_kernel's cap: on W [14336x4096] 1024 workgroups (4 per CU) encode 2% faster than 2048 or
// 4096 (0.0434-0.0436 against 0.0443-0.0447 ms per call from HBM), where row1d_kernel is fastest at
// 2048 (X [8192x4096]: 0.0270 against 0.0280 ms at 1024)
constexpr uint32_t kPass2Grid2D = 1024;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---- loads ----------------------------------------------------------------------------------------
// 16 consecutive elements (32 B bf16 / 64 B f32) kept raw.
template <int ESZ>
struct Raw16 {
  uint4 v[ESZ];
};

template <int ESZ>
__device__ __forceinline__ Raw16<ESZ> load_raw16(const uint8_t *__restrict__ p) {
  Raw16<ESZ> r;
#pragma unroll
  for (int i = 0; i < ESZ; ++i) r.v[i] = *reinterpret_cast<const uint4 *>(p + 16 * i);
  return r;
}

template <int ESZ>
__device__ __forceinline__ void unpack16(const Raw16<ESZ> &r, float (&y)[16]) {
#pragma unroll
  for (int i = 0; i < ESZ; ++i) {
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ESZ == 2) {
        y[8 * i + 2 * j] = bf16_lo(w[j]);
        y[8 * i + 2 * j + 1] = bf16_hi(w[j]);
      } else {
        y[4 * i + j] = __uint_as_float(w[j]);
      }
    }
  }
}

// rht16 (nvfp4_device.hpp) in two parts: the random signs D are applied while unpacking
// (unpack16_signed, rawn_elem_signed), then the butterfly below, with the 1/4 left to the caller
// when SCALE is false.  Same operations in the same order as rht16.
template <bool SCALE = true>
__device__ __forceinline__ void rht16_butterfly(float (&u)[16]) {
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
  if constexpr (SCALE) {
#pragma unroll
    for (int t = 0; t < 16; ++t) u[t] = u[t] * 0.25f;
  }
}

// unpack16 with the Hadamard transform's random signs applied (bit t of sign_word flips element t);
// the low bf16 half takes its flip as an addition of 2^31 (see rawn_elem_signed).
template <int ESZ>
__device__ __forceinline__ void unpack16_signed(const Raw16<ESZ> &r, float (&y)[16], uint32_t sign_word) {
#pragma unroll
  for (int i = 0; i < ESZ; ++i) {
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ESZ == 2) {
        const int t = 8 * i + 2 * j;
        y[t] = __uint_as_float((w[j] << 16) + (((sign_word >> t) & 1u) << 31));
        y[t + 1] = __uint_as_float((w[j] & 0xFFFF0000u) ^ (((sign_word >> (t + 1)) & 1u) << 31));
      } else {
        const int t = 4 * i + j;
        y[t] = __uint_as_float(w[j] ^ (((sign_word >> t) & 1u) << 31));
      }
    }
  }
}

// N consecutive elements at p (2N bytes of bf16 / 4N of f32, N = 4 or 8) kept raw, loaded 8 or 16
// bytes at a time.
template <int ESZ, int N = 8>
struct RawN {
  static constexpr int kBytes = N * ESZ;
  typedef typename std::conditional<kBytes == 8, uint2, uint4>::type Vec;
  Vec v[kBytes >= 16 ? kBytes / 16 : 1];
};
template <int ESZ>
using Raw8 = RawN<ESZ, 8>;

template <int ESZ, int N = 8>
__device__ __forceinline__ RawN<ESZ, N> loadn(const uint8_t *__restrict__ p) {
  RawN<ESZ, N> r;
  typedef typename RawN<ESZ, N>::Vec Vec;
#pragma unroll
  for (int i = 0; i < (N * ESZ >= 16 ? N * ESZ / 16 : 1); ++i) r.v[i] = *reinterpret_cast<const Vec *>(p + 16 * i);
  return r;
}

// 32-bit word q of a raw group (constant q after unrolling)
template <int ESZ, int N>
__device__ __forceinline__ uint32_t rawn_word(const RawN<ESZ, N> &r, int q) {
  if constexpr (N * ESZ == 8) {
    return q == 0 ? r.v[0].x : r.v[0].y;
  } else {
    const uint4 &x = r.v[q >> 2];
    return (q & 3) == 0 ? x.x : (q & 3) == 1 ? x.y : (q & 3) == 2 ? x.z : x.w;
  }
}

template <int ESZ, int N = 8>
__device__ __forceinline__ float rawn_elem(const RawN<ESZ, N> &r, int c) {
  if constexpr (ESZ == 2) {
    const uint32_t w = rawn_word<ESZ, N>(r, c >> 1);
    return (c & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    return __uint_as_float(rawn_word<ESZ, N>(r, c));
  }
}

// Element c with its sign flipped when sflip (0 or 2^31) is set: the random signs D of the Hadamard
// transform applied while unpacking.  For the low bf16 half, adding 2^31 to w << 16 flips its top
// bit (the carry leaves the word), one shift-and-add instead of a shift and an exclusive or.
template <int ESZ, int N>
__device__ __forceinline__ float rawn_elem_signed(const RawN<ESZ, N> &r, int c, uint32_t sflip) {
  if constexpr (ESZ == 2) {
    const uint32_t w = rawn_word<ESZ, N>(r, c >> 1);
    return (c & 1) ? __uint_as_float((w & 0xFFFF0000u) ^ sflip) : __uint_as_float((w << 16) + sflip);
  } else {
    return __uint_as_float(rawn_word<ESZ, N>(r, c) ^ sflip);
  }
}

template <int ESZ>
__device__ __forceinline__ float raw8_elem(const Raw8<ESZ> &r, int c) {
  return rawn_elem<ESZ, 8>(r, c);
}

// ---- element codes --------------------------------------------------------------------------------
// Stochastic rounding of 8 values y[t] * e on the hardware converter (v_cvt_scalef32_sr_pk_fp4_f32),
// element t drawing the 16 bits r16 of Philox word t >> 1, half t & 1.
//
// What the instruction does with its first element (measured on MI355X over 10^6 random inputs, then
// checked against the software rule below on every r16 for boundary-centred values in all seven
// grid intervals): with x = the fraction of |src| / 2^exp(scale) between its two E2M1 neighbours in
// units of 2^-22, it rounds up iff x + (seed >> 10) >= 2^22; from 6 up it gives 6; the sign is
// copied.  (Its second element reads seed bits 30..9, the same random value shifted by one bit, so
// only the first element of each instruction is used: one value per instruction.)
// The format's rule is: round up iff r16 < x / 64.  With seed bits 31..10 equal to
// 2^22 - 1 - 64 r16, i.e. seed = ~(r16 << 16) | 0xFFFF, the instruction rounds up iff
// x >= 64 r16 + 1, which is the format's rule whenever x is an integer.  x is an integer from 1 up
// (22 fraction bits); below 1 it may not be, so the value is first rounded up to a multiple of
// 2^-23: src = ceil(RN(|y| e) * 2^23) with the sign of y and scale 2^23 (an exact integer from
// 1 up, where it changes nothing; below 1, x > 64 r16 iff ceil(x) > 64 r16).
typedef float f32x2 __attribute__((ext_vector_type(2)));
// The instruction writes only the selected byte of its destination and keeps the other three
// (measured), but the compiler's builtin for it does not tie its first operand to the destination,
// so bytes accumulated through the builtin are lost; the instruction is therefore issued here with
// the accumulated word as a tied operand.
// FIRST: the accumulator's first conversion (byte 0).  The four conversions into one accumulator
// write all four bytes, so the first needs no initial value: its operand is output-only.
template <int SEL, bool FIRST = false>
__device__ __forceinline__ uint32_t cvt_sr_byte(uint32_t acc, float x, uint32_t seed) {
  const f32x2 src = {x, 0.0f};
  const float scale = 8388608.0f;  // 2^23: the instruction converts x / 2^23
  if constexpr (FIRST) {
    static_assert(SEL == 0, "the first conversion writes byte 0");
    uint32_t out;
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "=v"(out) : "v"(src), "v"(seed), "v"(scale));
    return out;
  } else if constexpr (SEL == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(src), "v"(seed), "v"(scale));
  else if constexpr (SEL == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(src), "v"(seed), "v"(scale));
  else if constexpr (SEL == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(src), "v"(seed), "v"(scale));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(src), "v"(seed), "v"(scale));
  return acc;
}

template <int T>  // element T of 8; nw = ~(its Philox word)
__device__ __forceinline__ void sr_elem(float y, float e, uint32_t nw, uint32_t &even, uint32_t &odd) {
  const float xs = __builtin_copysignf(__builtin_ceilf((fabsf(y) * e) * 8388608.0f), y);
  if constexpr ((T & 1) != 0)  // r16 = high half of the word
    odd = cvt_sr_byte<(T >> 1), T == 1>(odd, xs, nw | 0xFFFFu);
  else  // r16 = low half of the word
    even = cvt_sr_byte<(T >> 1), T == 0>(even, xs, (nw << 16) | 0xFFFFu);
}

__device__ __forceinline__ uint32_t pack8_sr(const float *y, float e, const u32x4 &w) {
  uint32_t even, odd;  // codes of even / odd elements in the low nibble of byte T >> 1
  const uint32_t n0 = ~w.x, n1 = ~w.y, n2 = ~w.z, n3 = ~w.w;
  sr_elem<0>(y[0], e, n0, even, odd);
  sr_elem<1>(y[1], e, n0, even, odd);
  sr_elem<2>(y[2], e, n1, even, odd);
  sr_elem<3>(y[3], e, n1, even, odd);
  sr_elem<4>(y[4], e, n2, even, odd);
  sr_elem<5>(y[5], e, n2, even, odd);
  sr_elem<6>(y[6], e, n3, even, odd);
  sr_elem<7>(y[7], e, n3, even, odd);
  return even | (odd << 4);
}

// ~(w << 16), the random operand of an even element (r16 = low half of w), in one instruction:
// sign-extended low 24 bits of w times -2^16 is -(w << 16) modulo 2^32, minus 1 is its complement.
__device__ __forceinline__ uint32_t seed_low_half(uint32_t w) {
  uint32_t r;
  asm("v_mad_i32_i24 %0, %1, %2, -1" : "=v"(r) : "v"(w), "s"(-65536));
  return r;
}

// Stochastic rounding with the 2^23 pre-scale folded into the block factor: the instruction's
// operand is ceil(RN(|y| * E)) with the sign of y, E = e * 2^23, or E = e * 2^21 when y holds four
// times the values to encode (the Hadamard transform's 1/4 left out).  encode_block_sr states when
// this equals the operand of sr_elem.
template <int T>  // element T of 8; w = its Philox word
__device__ __forceinline__ void sr_elem_folded(float y, float E, uint32_t w, uint32_t &even, uint32_t &odd) {
  const float xs = __builtin_copysignf(__builtin_ceilf(fabsf(y) * E), y);
  if constexpr ((T & 1) != 0)
    odd = cvt_sr_byte<(T >> 1), T == 1>(odd, xs, ~w | 0xFFFFu);
  else
    even = cvt_sr_byte<(T >> 1), T == 0>(even, xs, seed_low_half(w));
}

__device__ __forceinline__ uint32_t pack8_sr_folded(const float *y, float E, const u32x4 &w) {
  uint32_t even, odd;
  sr_elem_folded<0>(y[0], E, w.x, even, odd);
  sr_elem_folded<1>(y[1], E, w.x, even, odd);
  sr_elem_folded<2>(y[2], E, w.y, even, odd);
  sr_elem_folded<3>(y[3], E, w.y, even, odd);
  sr_elem_folded<4>(y[4], E, w.z, even, odd);
  sr_elem_folded<5>(y[5], E, w.z, even, odd);
  sr_elem_folded<6>(y[6], E, w.w, even, odd);
  sr_elem_folded<7>(y[7], E, w.w, even, odd);
  return even | (odd << 4);
}

// Decoded error terms of one byte of packed codes (two elements, low nibble first) under scale S:
// the decoded value is RN(RN(q * S) * ts), where q * S is exact (q has at most two significant bits,
// S four, and the product stays normal).  v_cvt_scalef32_pk_f32_fp4 with scale 1.0 returns the two
// E2M1 values q exactly, so each element costs half a conversion and two multiplies.
template <int BYTE>
__device__ __forceinline__ float sse_pair(uint32_t w, float y0, float y1, float S, float ts, float acc) {
  const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, BYTE);
  const float d0 = y0 - (q[0] * S) * ts;
  acc = fmaf(d0, d0, acc);
  const float d1 = y1 - (q[1] * S) * ts;
  return fmaf(d1, d1, acc);
}

// Packed codes of one 16-element block under factor e.  i0 = logical index of y[0] (a multiple of
// 16), used for the stochastic-rounding counter.
template <int MODE>
__device__ __forceinline__ void block_words(const float (&y)[16], float e, uint64_t i0, uint32_t key0, uint32_t key1,
                                            uint32_t stream_id, uint32_t &w0, uint32_t &w1) {
  auto degenerate = [&]() {
    w0 = 0u;
    w1 = 0u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      w0 |= code_degenerate(y[t]) << (4 * t);
      w1 |= code_degenerate(y[8 + t]) << (4 * t);
    }
  };
  if constexpr (MODE == kSR) {
    if (__builtin_isinf(e)) {
      degenerate();
    } else {
      const uint64_t call = i0 >> 3;
      const u32x4 r0 = philox4x32_10(static_cast<uint32_t>(call), static_cast<uint32_t>(call >> 32), stream_id, 0u,
                                     key0, key1);
      const u32x4 r1 = philox4x32_10(static_cast<uint32_t>(call + 1), static_cast<uint32_t>((call + 1) >> 32),
                                     stream_id, 0u, key0, key1);
      w0 = pack8_sr(y, e, r0);
      w1 = pack8_sr(y + 8, e, r1);
    }
  } else {
    // The conversion runs for every lane (an infinite factor gives undefined codes, replaced below);
    // the rare infinite factor (S * ts underflowed) is patched under a wave-uniform branch, so that
    // its per-element selects are not computed for every block (left to itself the compiler
    // computed them unconditionally for the second candidate of the Four-over-Six encode).
    w0 = pack8_rne(y, e);
    w1 = pack8_rne(y + 8, e);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(__builtin_isinf(e)) != 0, 0)) {
      if (__builtin_isinf(e)) degenerate();
    }
  }
}

// fp32 squared error of a block against its decoded codes, accumulated with fma in block order.
__device__ __forceinline__ float block_sse(const float (&y)[16], uint32_t w0, uint32_t w1, float S, float ts) {
  float acc = 0.0f;
  acc = sse_pair<0>(w0, y[0], y[1], S, ts, acc);
  acc = sse_pair<1>(w0, y[2], y[3], S, ts, acc);
  acc = sse_pair<2>(w0, y[4], y[5], S, ts, acc);
  acc = sse_pair<3>(w0, y[6], y[7], S, ts, acc);
  acc = sse_pair<0>(w1, y[8], y[9], S, ts, acc);
  acc = sse_pair<1>(w1, y[10], y[11], S, ts, acc);
  acc = sse_pair<2>(w1, y[12], y[13], S, ts, acc);
  return sse_pair<3>(w1, y[14], y[15], S, ts, acc);
}

// ---- stochastic rounding: per-workgroup tables and reciprocal divisions ---------------------------
// RN(a / b) from y = RN(1 / b): q = RN(a y) is within two ulps of a / b; one residual correction
// (r = a - q b by fma) makes it faithful, and a second one, whose residual is then exact, gives
// the correctly rounded quotient (Markstein's theorem: y within half an ulp of 1 / b, q within one
// ulp of a / b).  Valid while a, b, the quotient and the residuals are normal: the callers keep
// a in [2^-90, 2^100] (or 0) and b in [2^-100, 2^100].  Checked against IEEE division on the CPU
// for b = 6 and every a in [2^-90, 2^100], and for 2000 random b with 10^6 a each.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
  float q = a * y;
  float r = fmaf(-q, b, a);
  q = fmaf(r, y, q);
  r = fmaf(-q, b, a);
  return fmaf(r, y, q);
}

constexpr float kRecip6 = 0x1.555556p-3f;  // RN(1 / 6)
// RN(1 / T) for the search targets 5.5, 5, 4.5, 4
constexpr float kRecipTargets[5] = {0x1.555556p-3f, 0x1.745d18p-3f, 0x1.99999ap-3f, 0x1.c71c72p-3f, 0x1p-2f};

// Scale byte of a block with maximum ab (target 6), as block_scale computes it.  With ts in
// [2^-100, 2^100] (recip_ok; yts = RN(1 / ts)) and ab = 0 or in [2^-90, 2^100], both divisions go
// through div_by_recip: RN(ab / 6) is then normal, and RN(q / ts) is correctly rounded wherever it
// is normal; where it is not (below 2^-126) both forms are far below 2^-10, the smallest value
// that rounds to a nonzero scale, so the byte is 0 either way.
// Target T (yT = RN(1 / T)) for the Four-over-Six and search candidates: the same with ab / T.
__device__ __forceinline__ uint32_t block_scale_byte(float ab, float ts, float yts, bool recip_ok, float T = 6.0f,
                                                     float yT = kRecip6) {
  float S;
  if (recip_ok && (ab == 0.0f || (ab >= 0x1p-90f && ab <= 0x1p100f))) {
    const float q = div_by_recip(ab, T, yT);
    const float sc = fminf(div_by_recip(q, ts, yts), 448.0f);
    return e4m3_rne(sc, S);
  }
  return block_scale(ab, T, ts, S);
}

// Per-workgroup tables of the 127 scale bytes a block can get (s <= 448 rounds to at most 0x7E):
// e[b] = encode_factor(S(b), ts), and E[b] = the factor the shortcut encode multiplies by where it
// applies to that factor, else -1:
//   stochastic rounding: e * 2^23 (e * 2^21 with the quarter folded), encode_block_sr;
//   nearest-even: e, or e / 4 with the Hadamard quarter folded (bf16), encode_block_rne_tab;
//   Four-over-Six and the scale search: the decoded scale S(b) (encode_block_tab).
struct FactorTables {
  float e[128];
  float E[128];
};

template <int MODE, int ESZ, bool QUARTER>
__device__ __forceinline__ void build_factor_tables(FactorTables &t, float ts) {
  if (threadIdx.x < 128) {
    const uint32_t b = threadIdx.x;
    const float S = b < 8 ? static_cast<float>(b) * 0.001953125f
                          : __uint_as_float((((b >> 3) + 120u) << 23) | ((b & 7u) << 20));
    const float e = encode_factor(S, ts);
    bool fold;
    float E;
    if constexpr (MODE == kSR) {
      constexpr float kMinFactor = ESZ == 2 ? 0x1p-14f : 1.0f;
      fold = e == 0.0f || (e >= kMinFactor && e <= 0x1p100f);
      E = e * (QUARTER ? 0x1p21f : 0x1p23f);
    } else if constexpr (MODE == kFourOverSix || MODE == kSearch) {
      fold = true;  // E holds the decoded scale S(b) itself
      E = S;
    } else {
      // e / 4 is exact from 2^-124 up; RN(y e) of y = u / 4 (exact for bf16) is then RN(u (e / 4))
      fold = e == 0.0f || (e < __builtin_inff() && (!QUARTER || e >= 0x1p-124f));
      E = QUARTER ? e * 0.25f : e;
    }
    t.e[b] = e;
    t.E[b] = fold ? E : -1.0f;
  }
  __syncthreads();
}

// Stochastic-rounding encode of one 1D block of y' = y (QUARTER: y' = y / 4, y the Hadamard
// transform without its 1/4), as encode_block<kSR> of y'.  With v = RN(|y'| e), sr_elem feeds the
// instruction ceil(RN(v * 2^23)); the folded form feeds ceil(RN(|y'| e 2^23)), one rounding of the
// same product scaled by a power of two.  The two agree
//   - where v is normal: scaling by 2^23 commutes with rounding;
//   - where v is subnormal or zero: both operands are below 1 before the ceil, so both are 1 for a
//     product that rounds to a nonzero value and 0 otherwise, and the two products round to zero
//     together as long as |y'| e > 2^-150 for every nonzero y'.  Nonzero bf16 values, and the
//     quarters of their transforms, are at least 2^-135 (multiples of 2^-135: the inputs are
//     multiples of 2^-133 and so are all fp32 sums and differences of them), so e >= 2^-14 suffices;
//     nonzero fp32 values are at least 2^-149, so e >= 1 (no fold of the quarter: y / 4 may round);
//   - for e = 0 (a zero block scale): both are 0 (y' finite) or the same NaN;
//   - and E = e 2^23 stays finite for e <= 2^100.
// Other factors (inf: S * ts underflowed; NaN) take the unfolded path.  The factor of each scale
// byte, and whether it folds, come from the workgroup's tables (build_factor_tables).
template <int ESZ, bool QUARTER>
__device__ __forceinline__ void encode_block_sr(float (&y)[16], float ts, float yts, bool recip_ok,
                                                const FactorTables &tab, uint64_t i0, uint32_t key0, uint32_t key1,
                                                uint32_t stream_id, uint32_t &sbyte, uint32_t &w0, uint32_t &w1) {
  static_assert(ESZ == 2 || !QUARTER, "the quarter of an fp32 transform may round");
  float ab = block_absmax(y);
  if constexpr (QUARTER) ab = ab * 0.25f;  // = max RN(|y| / 4): rounding is monotone
  sbyte = block_scale_byte(ab, ts, yts, recip_ok);
  const float E = tab.E[sbyte];
  const uint64_t call = i0 >> 3;
  const u32x4 r0 = philox4x32_10(static_cast<uint32_t>(call), static_cast<uint32_t>(call >> 32), stream_id, 0u,
                                 key0, key1);
  const u32x4 r1 = philox4x32_10(static_cast<uint32_t>(call + 1), static_cast<uint32_t>((call + 1) >> 32),
                                 stream_id, 0u, key0, key1);
  if (E >= 0.0f) {
    w0 = pack8_sr_folded(y, E, r0);
    w1 = pack8_sr_folded(y + 8, E, r1);
  } else {
    const float e = tab.e[sbyte];
    if constexpr (QUARTER) {
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = y[t] * 0.25f;  // in place: y is not read after the encode
    }
    if (__builtin_isinf(e)) {
      w0 = 0u;
      w1 = 0u;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        w0 |= code_degenerate(y[t]) << (4 * t);
        w1 |= code_degenerate(y[8 + t]) << (4 * t);
      }
    } else {
      w0 = pack8_sr(y, e, r0);
      w1 = pack8_sr(y + 8, e, r1);
    }
  }
}

// Nearest-even encode of one 1D block of y' = y (QUARTER: y' = y / 4), as encode_block<kRNE> of y':
// scale byte through reciprocals (block_scale_byte), factor from the tables, codes of RN(y E).
template <int ESZ, bool QUARTER>
__device__ __forceinline__ void encode_block_rne_tab(float (&y)[16], float ts, float yts, bool recip_ok,
                                                     const FactorTables &tab, uint32_t &sbyte, uint32_t &w0,
                                                     uint32_t &w1) {
  static_assert(ESZ == 2 || !QUARTER, "the quarter of an fp32 transform may round");
  float ab = block_absmax(y);
  if constexpr (QUARTER) ab = ab * 0.25f;  // = max RN(|y| / 4): rounding is monotone
  sbyte = block_scale_byte(ab, ts, yts, recip_ok);
  const float E = tab.E[sbyte];
  if (E >= 0.0f) {
    w0 = pack8_rne(y, E);
    w1 = pack8_rne(y + 8, E);
  } else {
    const float e = tab.e[sbyte];
    if constexpr (QUARTER) {
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = y[t] * 0.25f;
    }
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
}

// Full encode of one 1D block: scale byte and two packed words (nibble t at bits 4t).  With
// Four-over-Six (targets 6, 4) or the scale search (6, 5.5, 5, 4.5, 4) every target gives a scale
// and codes; the block keeps the lowest squared error, a later target only if strictly lower.
template <int MODE>
__device__ __forceinline__ void encode_block(const float (&y)[16], float ab, float ts, uint64_t i0, uint32_t key0,
                                             uint32_t key1, uint32_t stream_id, uint32_t &sbyte, uint32_t &w0,
                                             uint32_t &w1) {
  float S;
  sbyte = block_scale(ab, 6.0f, ts, S);
  block_words<MODE>(y, encode_factor(S, ts), i0, key0, key1, stream_id, w0, w1);
  if constexpr (MODE == kFourOverSix || MODE == kSearch) {
    constexpr int NT = MODE == kSearch ? 5 : 2;
    float best = block_sse(y, w0, w1, S, ts);
#pragma unroll
    for (int ti = 1; ti < NT; ++ti) {
      const float T = MODE == kSearch ? 6.0f - 0.5f * ti : 4.0f;  // 5.5, 5, 4.5, 4 (exact)
      float Sx;
      const uint32_t sbx = block_scale(ab, T, ts, Sx);
      uint32_t v0, v1;
      block_words<kRNE>(y, encode_factor(Sx, ts), i0, key0, key1, stream_id, v0, v1);
      const float acc = block_sse(y, v0, v1, Sx, ts);
      if (acc < best) {
        best = acc;
        sbyte = sbx;
        w0 = v0;
        w1 = v1;
      }
    }
  }
}


// encode_block<kFourOverSix / kSearch> with the candidates' scale bytes through reciprocals
// (block_scale_byte) and their factors e and decoded scales S from the workgroup's tables: the same
// candidates, codes and errors, so the same choice.
template <int MODE>
__device__ __forceinline__ void encode_block_tab(const float (&y)[16], float ts, float yts, bool recip_ok,
                                                 const FactorTables &tab, uint32_t &sbyte, uint32_t &w0,
                                                 uint32_t &w1) {
  static_assert(MODE == kFourOverSix || MODE == kSearch, "candidate modes only");
  const float ab = block_absmax(y);
  sbyte = block_scale_byte(ab, ts, yts, recip_ok);
  block_words<kRNE>(y, tab.e[sbyte], 0u, 0u, 0u, 0u, w0, w1);
  constexpr int NT = MODE == kSearch ? 5 : 2;
  float best = block_sse(y, w0, w1, tab.E[sbyte], ts);
#pragma unroll
  for (int ti = 1; ti < NT; ++ti) {
    const int k = MODE == kSearch ? ti : 4;  // index of T in 6, 5.5, 5, 4.5, 4
    const uint32_t sbx = block_scale_byte(ab, ts, yts, recip_ok, 6.0f - 0.5f * k, kRecipTargets[k]);
    uint32_t v0, v1;
    block_words<kRNE>(y, tab.e[sbx], 0u, 0u, 0u, 0u, v0, v1);
    const float acc = block_sse(y, v0, v1, tab.E[sbx], ts);
    if (acc < best) {
      best = acc;
      sbyte = sbx;
      w0 = v0;
      w1 = v1;
    }
  }
}

// Workgroup max of one value per lane -> partial[blockIdx.x] (thread 0).  NT = threads per group.
template <uint32_t NT = kThreads>
__device__ __forceinline__ void write_partial(uint32_t m, uint32_t *__restrict__ partial) {
  __shared__ uint32_t red[NT / 64];
  m = wave_max_u32(m);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (uint32_t w = 1; w < NT / 64; ++w) r = max(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// The maximum of RN(|u| / 4) over values whose largest |u| has the float bits m: rounding is
// monotone, so the maximum of the quartered values is the quartered maximum (pass 1 of the Hadamard
// variants takes the 1/4 of the transform once per lane instead of once per element).
__device__ __forceinline__ uint32_t quarter_bits(uint32_t m) { return __float_as_uint(__uint_as_float(m) * 0.25f); }

// Tensor amax from the pass-1 partial maxima (float bits of non-negative values compare like
// unsigned integers), reduced by every wave on its own (at most kPass1Parts values, no barrier);
// ts = amax / ts_div; wave 0 of workgroup 0 publishes ts.
__device__ __forceinline__ float tensor_scale(const uint32_t *__restrict__ partial, uint32_t nparts,
                                              float *__restrict__ ts_out, float ts_div) {
  const uint32_t lane = threadIdx.x & 63u;
  uint32_t m = 0;
#pragma unroll 4
  for (uint32_t i = lane; i < nparts; i += 64) m = max(m, partial[i]);
  m = wave_max_u32(m);
  const float ts = __uint_as_float(m) / ts_div;  // 2688 (6 * 448), or 1792 (4 * 448)
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = ts;
  return ts;
}

// ---- groups ------------------------------------------------------------------------------------------
// A grouped call (grid dimension y = group g) quantizes G equally shaped tensors in one launch per
// pass: group g reads x + g * x bytes, writes its codes and scale bytes at g times the per-group
// sizes and its tensor scale to ts_out[g], keeps its pass-1 maxima at partial + g * (pass-1
// workgroups), and draws its stochastic rounding from stream stream_id + g.  That is exactly what a
// separate call on the group's tensor with stream id stream_id + g computes.
struct GroupStrides {
  int64_t x, data, scales;  // bytes per group
};

template <class A>
__device__ __forceinline__ void enter_group(A &p, uint32_t parts) {
  const uint32_t g = blockIdx.y;
  p.x += g * p.g.x;
  p.data += g * p.g.data;
  p.scales += g * p.g.scales;
  p.ts_out += g;
  p.partial += static_cast<int64_t>(g) * parts;
}

// ---- pass 1: plain tensor amax ----------------------------------------------------------------------
struct AmaxArgs {
  const uint8_t *x;
  int64_t ldx_bytes;
  uint32_t total_chunks;  // 16-byte chunks
  FastDiv cpr;            // chunks per row
  uint32_t flat;          // rows are contiguous (ldx == row length)
  uint32_t *partial;
  int64_t g_x;            // bytes between the inputs of consecutive groups (grid dimension y)
  // 16-row bands for the 2D encode: a band is band_p slabs of 1024 chunks (band_p in 1, 2, 4, ..., 32,
  // 256 workgroups), or 0
  uint32_t band_p;
};

template <int ESZ>
__device__ __forceinline__ void absmax_chunk(const uint4 &v, u16x2 &m2, uint32_t &m4) {
  if constexpr (ESZ == 2) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
  } else {
    m4 = max(m4, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
  }
}

template <int ESZ>
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(AmaxArgs p) {
  // Four 16-byte loads in flight per lane, and the remaining (< U) chunks of a lane issued together
  // with clamped indices (a repeated chunk leaves a maximum unchanged): eight per lane, or a tail
  // read one chunk at a time, measured 5-10% slower on inputs streamed from HBM.
  constexpr int U = 4;
  p.x += blockIdx.y * p.g_x;
  p.partial += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  const uint32_t stride = gridDim.x * kAmaxThreads;
  u16x2 m2 = {0, 0};
  uint32_t m4 = 0;
  auto addr = [&](uint32_t c) -> const uint4 * {
    if (p.flat) return reinterpret_cast<const uint4 *>(p.x) + c;
    const uint32_t r = fdiv(c, p.cpr);
    return reinterpret_cast<const uint4 *>(p.x + static_cast<int64_t>(r) * p.ldx_bytes +
                                           static_cast<int64_t>(c - r * p.cpr.d) * 16);
  };
  // Workgroup w reads slab vw of each grid step (slab = 1024 chunks).  With 16-row bands of band_p
  // slabs, vw relabels the workgroups so that the slabs of band b are read on XCD b mod 8 (workgroup
  // w runs on XCD w mod 8): w = 8 g + x reads band 8 (g / band_p) + x of the step's bands, slab
  // g mod band_p of it.  A bijection of the step's 256 slabs, so every chunk is read once.
  uint32_t vw = blockIdx.x;
  if (p.band_p != 0) {
    const uint32_t g = blockIdx.x >> 3, x = blockIdx.x & 7u;
    vw = p.band_p * (8u * (g / p.band_p) + x) + g % p.band_p;
  }
  uint32_t c = vw * kAmaxThreads + threadIdx.x;
  for (; c + (U - 1) * stride < p.total_chunks; c += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *addr(c + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) absmax_chunk<ESZ>(v[u], m2, m4);
  }
  if (c < p.total_chunks) {
    uint4 v[U - 1];
#pragma unroll
    for (int u = 0; u < U - 1; ++u) v[u] = *addr(min(c + u * stride, p.total_chunks - 1));
#pragma unroll
    for (int u = 0; u < U - 1; ++u) absmax_chunk<ESZ>(v[u], m2, m4);
  }
  const uint32_t m = ESZ == 2 ? (static_cast<uint32_t>(max(m2.x, m2.y)) << 16) : m4;
  write_partial<kAmaxThreads>(m, p.partial);
}

// ---- ROW mode, 1D blocks ----------------------------------------------------------------------------
struct RowArgs {
  const uint8_t *x;
  int64_t ldx_bytes;
  uint32_t nblocks;  // R * K / 16
  FastDiv kb;        // blocks per row, K / 16
  int64_t K;
  const uint32_t *partial;
  uint32_t nparts;
  uint32_t *partial_out;
  uint8_t *data;
  uint8_t *scales;
  float *ts_out;
  uint32_t key0, key1, stream_id, sign_word;
  float *rht_out;
  float ts_div;
  GroupStrides g;
  // Pass 2 only: the pass-1 slab (blocks one pass-1 workgroup read per grid step; its XCD is the slab
  // index mod 8), or 0 for the plain grid-stride order.
  uint32_t slab;
};

// The blocks one lane of row1d_kernel encodes, in order: slab s_k = s0 + ds k (k < ns) of Z blocks,
// piece h < H of 256 blocks (one per lane) within it.  Plain order: Z = 256, s0 = workgroup, ds =
// grid.  XCD order (pass 2 after a pass 1 whose workgroups read slab s on XCD s mod 8): workgroup w
// (on XCD w mod 8) walks the slabs of its own XCD, the last-read slab first.  Measured faster than
// the plain order, the plain order reversed and the XCD order walked forwards, none of which differ
// from one another; the L2 serves none of the re-reads (the same bytes are fetched from beyond it in
// every order), so the gain is in how the reads meet the Infinity Cache and HBM.
struct BlockOrder {
  int32_t s0, ds;
  uint32_t nq, Z, lh;  // nq = ns * H, H = 1 << lh
  __device__ __forceinline__ uint32_t block(uint32_t q) const {
    return static_cast<uint32_t>(s0 + ds * static_cast<int32_t>(q >> lh)) * Z + (q & ((1u << lh) - 1u)) * 256u +
           threadIdx.x;
  }
};

__device__ __forceinline__ BlockOrder block_order(uint32_t n, uint32_t slab) {
  static_assert(kThreads == 256, "one block per lane per 256-block piece");
  BlockOrder o;
  const uint32_t w = blockIdx.x, grid = gridDim.x;
  if (slab == 0) {
    const uint32_t S = (n + 255u) / 256u;
    o.s0 = static_cast<int32_t>(w);
    o.ds = static_cast<int32_t>(grid);
    o.nq = w < S ? (S - 1u - w) / grid + 1u : 0u;
    o.Z = 256u;
    o.lh = 0;
  } else {
    const uint32_t x = w & 7u, k = w >> 3, g8 = grid >> 3;
    const uint32_t S = (n + slab - 1u) / slab, J = x < S ? (S - x + 7u) / 8u : 0u;
    const uint32_t lh = slab == 512u ? 1u : (slab == 1024u ? 2u : 0u);
    o.s0 = static_cast<int32_t>(x + 8u * (J - 1u - k));
    o.ds = -8 * static_cast<int32_t>(g8);
    o.nq = k < J ? ((J - 1u - k) / g8 + 1u) << lh : 0u;
    o.Z = slab;
    o.lh = lh;
  }
  return o;
}

template <int ESZ, int MODE, bool RHT, bool PASS1>
__global__ __launch_bounds__(kThreads) void row1d_kernel(RowArgs p) {
  enter_group(p, p.nparts);
  p.partial_out += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  p.stream_id += blockIdx.y;
  const BlockOrder order = block_order(p.nblocks, PASS1 ? 0u : p.slab);
  uint32_t q = 0;
  uint32_t b = order.nq > 0 ? order.block(0) : p.nblocks;  // (>= nblocks: not a block to encode)
  auto src = [&](uint32_t blk) {
    const uint32_t r = fdiv(blk, p.kb);
    return p.x + static_cast<int64_t>(r) * p.ldx_bytes + static_cast<int64_t>(blk - r * p.kb.d) * 16 * ESZ;
  };
  Raw16<ESZ> cur, nxt;
  if (b < p.nblocks) cur = load_raw16<ESZ>(src(b));
  float ts = 0.0f;
  if constexpr (!PASS1) ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  // stochastic rounding and 1D nearest-even of bf16 keep the transform's 1/4 out of the elements
  // (encode_block_sr, encode_block_rne_tab)
  constexpr bool QUARTER = RHT && (PASS1 || ((MODE == kSR || MODE == kRNE) && ESZ == 2));
  constexpr bool TABLES = !PASS1;  // every 1D mode
  __shared__ FactorTables tab;
  float yts = 0.0f;
  bool recip_ok = false;
  if constexpr (TABLES) {
    build_factor_tables<MODE, ESZ, QUARTER>(tab, ts);
    recip_ok = ts >= 0x1p-100f && ts <= 0x1p100f;
    yts = 1.0f / ts;
  }
  uint32_t mx = 0;
  for (; q < order.nq; ++q) {
    const uint32_t bn = q + 1 < order.nq ? order.block(q + 1) : p.nblocks;
    if (bn < p.nblocks) nxt = load_raw16<ESZ>(src(bn));
    if (b >= p.nblocks) {  // the top slab's missing blocks
      cur = nxt;
      b = bn;
      continue;
    }
    float y[16];
    if constexpr (RHT) {
      unpack16_signed<ESZ>(cur, y, p.sign_word);
      rht16_butterfly<!QUARTER>(y);
    } else {
      unpack16<ESZ>(cur, y);
    }
    if constexpr (PASS1) {
      mx = max(mx, __float_as_uint(block_absmax(y)));
    } else {
      const uint32_t r = fdiv(b, p.kb);
      const uint64_t i0 = static_cast<uint64_t>(r) * static_cast<uint64_t>(p.K) + 16u * (b - r * p.kb.d);
      if constexpr (RHT) {
        if (p.rht_out) {
          float4 *o = reinterpret_cast<float4 *>(p.rht_out + i0);
          float w[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            // opaque copy: the quarters stay in this branch (not hoisted as common with the encode's)
            w[t] = y[t];
            asm volatile("" : "+v"(w[t]));
            if constexpr (QUARTER) w[t] = w[t] * 0.25f;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
      }
      uint32_t sb, w0, w1;
      if constexpr (MODE == kSR)
        encode_block_sr<ESZ, QUARTER>(y, ts, yts, recip_ok, tab, i0, p.key0, p.key1, p.stream_id, sb, w0, w1);
      else if constexpr (MODE == kRNE)
        encode_block_rne_tab<ESZ, QUARTER>(y, ts, yts, recip_ok, tab, sb, w0, w1);
      else
        encode_block_tab<MODE>(y, ts, yts, recip_ok, tab, sb, w0, w1);
      *reinterpret_cast<uint2 *>(p.data + (i0 >> 1)) = make_uint2(w0, w1);
      p.scales[i0 >> 4] = static_cast<uint8_t>(sb);
    }
    cur = nxt;
    b = bn;
  }
  if constexpr (PASS1) write_partial(RHT ? quarter_bits(mx) : mx, p.partial_out);
}

// Nearest-even codes of 8 values under factor e (e = +inf: S * ts underflowed, see code_degenerate).
__device__ __forceinline__ uint32_t codes8(const float (&yv)[8], float e) {
  if (__builtin_isinf(e)) {
    uint32_t w = 0u;
#pragma unroll
    for (int c = 0; c < 8; ++c) w |= code_degenerate(yv[c]) << (4 * c);
    return w;
  }
  return pack8_rne(yv, e);
}

// ---- ROW mode, 16x16 tiles --------------------------------------------------------------------------
struct Row2dArgs {
  const uint8_t *x;
  int64_t ldx_bytes;
  uint32_t ntasks;  // (R / 16) * nseg
  FastDiv nseg;     // 512-column segments per 16-row band
  int64_t K;
  const uint32_t *partial;
  uint32_t nparts;
  uint8_t *data;
  uint8_t *scales;
  float *ts_out;
  float ts_div;
  GroupStrides g;
  // pass 1 left band b on XCD b mod 8 (AmaxArgs::band_p) and the grid is a multiple of 8: the waves
  // take the bands of their own XCD, last-read band first (the order of row1d_kernel's XCD order)
  uint32_t affine;
};

// An empty asm that claims to modify the patch's registers: values unpacked from it before are not
// reused after, the compiler unpacks again (one instruction per element) instead of holding them.
template <int ESZ, int N>
__device__ __forceinline__ void opaque_patch(RawN<ESZ, N> (&v)[16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int i = 0; i < (N * ESZ >= 16 ? N * ESZ / 16 : 1); ++i) {
      asm volatile("" : "+v"(v[t].v[i].x), "+v"(v[t].v[i].y));
      if constexpr (N * ESZ >= 16) asm volatile("" : "+v"(v[t].v[i].z), "+v"(v[t].v[i].w));
    }
}

template <int ESZ, int N = 8>
__device__ __forceinline__ void load_patch(RawN<ESZ, N> (&v)[16], const uint8_t *__restrict__ base, int64_t ld_bytes,
                                           bool valid) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (valid) {
      v[t] = loadn<ESZ, N>(base + t * ld_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < (N * ESZ >= 16 ? N * ESZ / 16 : 1); ++i) v[t].v[i] = {};
    }
  }
}

// ---- Four-over-Six on 16x16 tiles ----------------------------------------------------------------
// The tile error is the sum of the 256 rounded squares RN(d * d), d = y - RN(RN(q * S) * ts), over a
// quad tree: a 2n x 2n block is RN(RN(TL + BR) + RN(TR + BL)) of its four n x n blocks, down to
// single elements.  Transposing a tile keeps TL and BR and swaps TR with BL, so a tile and its
// transpose (row-wise and column-wise quantization) get the same error and the same choice.

// Rounded squared errors of two elements against their nearest-even codes under factor e / scale S.
__device__ __forceinline__ f32x2 sq_pair(float y0, float y1, float e, float S, float ts) {
  uint32_t w;
  if (__builtin_isinf(e))
    w = code_degenerate(y0) | (code_degenerate(y1) << 4);
  else
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0 * e, y1 * e, 1.0f, 0);
  const f32x2 q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float d0 = y0 - (q[0] * S) * ts, d1 = y1 - (q[1] * S) * ts;
  return f32x2{d0 * d0, d1 * d1};
}

// Quad-tree sum of the N x N block at (r, c); leaf(r, c) is the sum of the 2 x 2 block at (r, c),
// (p(r, c) + p(r+1, c+1)) + (p(r, c+1) + p(r+1, c)).
template <int N, class Leaf>
__device__ __forceinline__ float quad_sum(const Leaf &leaf, int r, int c) {
  if constexpr (N == 2) {
    return leaf(r, c);
  } else {
    constexpr int H = N / 2;
    const float diag = quad_sum<H>(leaf, r, c) + quad_sum<H>(leaf, r + H, c + H);
    const float off = quad_sum<H>(leaf, r, c + H) + quad_sum<H>(leaf, r + H, c);
    return diag + off;
  }
}

// Tile error for the lane pair of a row-wise 16x16 tile: lane holds tile rows 0-15 of columns 0-7
// (even lane) or 8-15 (odd lane), element (r, c) = column c of v[r].
template <int ESZ>
__device__ __forceinline__ float tile_sse_rows(const Raw8<ESZ> (&v)[16], float e, float S, float ts, bool even) {
  auto leaf = [&](int r, int c) {
    const f32x2 a = sq_pair(raw8_elem<ESZ>(v[r], c), raw8_elem<ESZ>(v[r], c + 1), e, S, ts);
    const f32x2 b = sq_pair(raw8_elem<ESZ>(v[r + 1], c), raw8_elem<ESZ>(v[r + 1], c + 1), e, S, ts);
    return (a[0] + b[1]) + (a[1] + b[0]);
  };
  const float top = quad_sum<8>(leaf, 0, 0), bottom = quad_sum<8>(leaf, 8, 0);
  const float top_o = __shfl_xor(top, 1, 64), bottom_o = __shfl_xor(bottom, 1, 64);
  const float tl = even ? top : top_o, tr = even ? top_o : top;
  const float bl = even ? bottom : bottom_o, br = even ? bottom_o : bottom;
  return (tl + br) + (tr + bl);
}

// Tile error for the lane pair of a column-wise 16x16 tile of Y = x^T: lane holds Y rows 0-7 (even
// lane) or 8-15 (odd lane) of Y columns (tokens) 0-15, element (r, k) = column r of v[k].
template <int ESZ>
__device__ __forceinline__ float tile_sse_cols(const Raw8<ESZ> (&v)[16], float e, float S, float ts, bool even) {
  auto leaf = [&](int r, int k) {
    const f32x2 a = sq_pair(raw8_elem<ESZ>(v[k], r), raw8_elem<ESZ>(v[k + 1], r), e, S, ts);
    const f32x2 b = sq_pair(raw8_elem<ESZ>(v[k], r + 1), raw8_elem<ESZ>(v[k + 1], r + 1), e, S, ts);
    return (a[0] + b[1]) + (a[1] + b[0]);
  };
  const float left = quad_sum<8>(leaf, 0, 0), right = quad_sum<8>(leaf, 0, 8);
  const float left_o = __shfl_xor(left, 1, 64), right_o = __shfl_xor(right, 1, 64);
  const float tl = even ? left : left_o, tr = even ? right : right_o;
  const float bl = even ? left_o : left, br = even ? right_o : right;
  return (tl + br) + (tr + bl);
}

template <int ESZ, bool FOS>
__global__ __launch_bounds__(kThreads) void row2d_kernel(Row2dArgs p) {
  enter_group(p, p.nparts);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const int64_t KB = p.K / 16;
  uint32_t task = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  // XCD order: XCD x owns bands x, x + 8, ...; its task (j, segment) is a segment of the XCD's
  // j-th band counted from the last (j = 0: the highest band x owns); this wave takes XCD-local
  // tasks v, v + 4 (grid / 8), ...
  const uint32_t xcd = blockIdx.x & 7u, nbands = p.ntasks / p.nseg.d;
  const uint32_t jx = xcd < nbands ? (nbands - xcd + 7u) / 8u : 0u;  // the XCD's bands
  const uint32_t ntasks_x = jx * p.nseg.d;
  if (p.affine) {
    task = ((blockIdx.x >> 3) * kThreads + threadIdx.x) >> 6;
  }
  const uint32_t ntasks = p.affine ? ntasks_x : p.ntasks;
  const uint32_t nwaves_x = p.affine ? (gridDim.x >> 3) * (kThreads / 64) : nwaves;
  Raw8<ESZ> v[16];
  auto start = [&](uint32_t tk, int64_t &r0, int64_t &c0) {
    uint32_t band, seg;
    if (p.affine) {
      const uint32_t j = fdiv(tk, p.nseg);
      band = xcd + 8u * (jx - 1u - j);
      seg = tk - j * p.nseg.d;
    } else {
      band = fdiv(tk, p.nseg);
      seg = tk - band * p.nseg.d;
    }
    r0 = static_cast<int64_t>(band) * 16;
    c0 = static_cast<int64_t>(seg) * 512 + lane * 8;
  };
  int64_t r0 = 0, c0 = 0;
  if (task < ntasks) {
    start(task, r0, c0);
    load_patch<ESZ>(v, p.x + r0 * p.ldx_bytes + c0 * ESZ, p.ldx_bytes, c0 < p.K);
  }
  const float ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  while (task < ntasks) {
    const bool valid = c0 < p.K;  // K % 16 == 0: both lanes of a tile agree
    float ab = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int c = 0; c < 8; ++c) ab = fmaxf(ab, fabsf(raw8_elem<ESZ>(v[t], c)));
    ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
    // unpack again below rather than keep all 128 values unpacked (which costs 128 registers)
    opaque_patch<ESZ, 8>(v);
    float S;
    uint32_t sb = block_scale(ab, 6.0f, ts, S);
    float e = encode_factor(S, ts);
    if constexpr (FOS) {
      // Four-over-Six on the tile: target 4 only if its tile error is strictly lower
      const bool even = (lane & 1u) == 0;
      const float sse6 = tile_sse_rows<ESZ>(v, e, S, ts, even);
      opaque_patch<ESZ, 8>(v);
      float S4;
      const uint32_t sb4 = block_scale(ab, 4.0f, ts, S4);
      const float e4 = encode_factor(S4, ts);
      const float sse4 = tile_sse_rows<ESZ>(v, e4, S4, ts, even);
      opaque_patch<ESZ, 8>(v);
      if (sse4 < sse6) {
        sb = sb4;
        e = e4;
      }
    }
    uint32_t w[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float yv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) yv[c] = raw8_elem<ESZ>(v[t], c);
      w[t] = codes8(yv, e);
    }
    const int64_t wr0 = r0, wc0 = c0;
    // next task's loads go out before this task's stores
    task += nwaves_x;
    if (task < ntasks) {
      start(task, r0, c0);
      load_patch<ESZ>(v, p.x + r0 * p.ldx_bytes + c0 * ESZ, p.ldx_bytes, c0 < p.K);
    }
    if (valid) {
#pragma unroll
      for (int t = 0; t < 16; ++t) *reinterpret_cast<uint32_t *>(p.data + (wr0 + t) * (p.K / 2) + wc0 / 2) = w[t];
      if ((lane & 1u) == 0) p.scales[(wr0 / 16) * KB + wc0 / 16] = static_cast<uint8_t>(sb);
    }
  }
}

// ---- COLWISE mode (1D blocks along x's dim 0, or 16x16 tiles) ------------------------------------------
struct ColArgs {
  const uint8_t *x;
  int64_t ldx_bytes;
  int64_t K;  // logical K = rows of x (tokens)
  int64_t R;  // logical R = cols of x
  uint32_t ntiles;
  FastDiv ntr;  // column tiles (128 columns each)
  const uint32_t *partial;
  uint32_t nparts;
  uint32_t *partial_out;
  uint8_t *data;
  uint8_t *scales;
  float *ts_out;
  uint32_t key0, key1, stream_id, sign_word;
  float *rht_out;
  float ts_div;
  GroupStrides g;
};

constexpr int kColTokens = 256;  // per workgroup tile

template <int ESZ, int MODE, bool RHT, bool B2D, bool ALIGNED, int CPL>
__global__ __launch_bounds__(kThreads) void col_kernel(ColArgs p) {
  static_assert(CPL == 8 || (CPL == 4 && !B2D), "16x16 tiles take a lane pair of 8 columns each");
  constexpr int COLS = 16 * CPL;  // columns of x (rows of Y) per workgroup tile
  enter_group(p, p.nparts);
  p.stream_id += blockIdx.y;
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[COLS * (kColTokens / 2)];
  __shared__ __attribute__((aligned(16))) uint8_t lds_scales[COLS * (kColTokens / 16)];
  const uint32_t ti = threadIdx.x >> 4;  // token group (16 tokens)
  const uint32_t tj = threadIdx.x & 15;  // column group (CPL columns)
  const int64_t KB = p.K / 16;
  RawN<ESZ, CPL> v[16];
  int64_t K0 = 0, R0 = 0, kk = 0, rr = 0;
  bool valid = false;
  auto locate = [&](uint32_t tile) {
    const uint32_t tk = fdiv(tile, p.ntr);
    K0 = static_cast<int64_t>(tk) * kColTokens;
    R0 = static_cast<int64_t>(tile - tk * p.ntr.d) * COLS;
    kk = K0 + 16 * ti;
    rr = R0 + CPL * tj;
    valid = kk < p.K && rr < p.R;  // K % 16 == 0 and R % 8 == 0
  };
  uint32_t tile = blockIdx.x;
  if (tile < p.ntiles) {
    locate(tile);
    load_patch<ESZ, CPL>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, valid);
  }
  const float ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  // stochastic rounding and 1D nearest-even of bf16 keep the transform's 1/4 out of the elements
  // (encode_block_sr, encode_block_rne_tab)
  constexpr bool QUARTER = RHT && (MODE == kSR || (MODE == kRNE && !B2D)) && ESZ == 2;
  constexpr bool TABLES = !B2D;  // every 1D mode
  uint32_t sflip[16];  // the transform's sign of token t: 0 or 2^31
#pragma unroll
  for (int t = 0; t < 16; ++t) sflip[t] = RHT ? ((p.sign_word >> t) & 1u) << 31 : 0u;
  __shared__ FactorTables tab;
  float yts = 0.0f;
  bool recip_ok = false;
  if constexpr (TABLES) {
    build_factor_tables<MODE, ESZ, QUARTER>(tab, ts);
    recip_ok = ts >= 0x1p-100f && ts <= 0x1p100f;
    yts = 1.0f / ts;
  }
  for (; tile < p.ntiles; tile += gridDim.x) {
    float S2d = 0.0f, e2d = 0.0f;
    uint32_t sb2d = 0;
    if constexpr (B2D) {
      float ab = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int c = 0; c < 8; ++c) ab = fmaxf(ab, fabsf(rawn_elem<ESZ, CPL>(v[t], c)));
      ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
      opaque_patch<ESZ, CPL>(v);  // unpack again below rather than hold 128 values
      sb2d = block_scale(ab, 6.0f, ts, S2d);
      e2d = encode_factor(S2d, ts);
      if constexpr (MODE == kFourOverSix) {
        // Four-over-Six on the tile: this lane holds 8 rows (top or bottom half) of the tile
        const bool even = (tj & 1u) == 0;
        const float sse6 = tile_sse_cols<ESZ>(v, e2d, S2d, ts, even);
        opaque_patch<ESZ, CPL>(v);
        float S4;
        const uint32_t sb4 = block_scale(ab, 4.0f, ts, S4);
        const float e4 = encode_factor(S4, ts);
        const float sse4 = tile_sse_cols<ESZ>(v, e4, S4, ts, even);
        opaque_patch<ESZ, CPL>(v);
        if (sse4 < sse6) {
          sb2d = sb4;
          S2d = S4;
          e2d = e4;
        }
      }
      if (valid && (tj & 1u) == 0) p.scales[(rr / 16) * KB + kk / 16] = static_cast<uint8_t>(sb2d);
    }
    uint64_t i0 = static_cast<uint64_t>(rr) * static_cast<uint64_t>(p.K) + static_cast<uint64_t>(kk);
#pragma unroll
    for (int c = 0; c < CPL; ++c, i0 += static_cast<uint64_t>(p.K)) {  // i0: logical index of (rr + c, kk)
      float u[16];
      if constexpr (RHT) {
#pragma unroll
        for (int t = 0; t < 16; ++t) u[t] = rawn_elem_signed<ESZ, CPL>(v[t], c, sflip[t]);
        rht16_butterfly<!QUARTER>(u);
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) u[t] = rawn_elem<ESZ, CPL>(v[t], c);
      }
      if constexpr (RHT) {
        if (p.rht_out && valid) {
          float4 *o = reinterpret_cast<float4 *>(p.rht_out + i0);
          float w[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            // opaque copy: the quarters stay in this branch (not hoisted as common with the encode's)
            w[t] = u[t];
            asm volatile("" : "+v"(w[t]));
            if constexpr (QUARTER) w[t] = w[t] * 0.25f;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
        }
      }
      uint32_t sb, w0, w1;
      if constexpr (B2D) {
        block_words<kRNE>(u, e2d, i0, 0u, 0u, 0u, w0, w1);
        sb = sb2d;
      } else if constexpr (MODE == kSR) {
        encode_block_sr<ESZ, QUARTER>(u, ts, yts, recip_ok, tab, i0, p.key0, p.key1, p.stream_id, sb, w0, w1);
      } else if constexpr (MODE == kRNE) {
        encode_block_rne_tab<ESZ, QUARTER>(u, ts, yts, recip_ok, tab, sb, w0, w1);
      } else {
        encode_block_tab<MODE>(u, ts, yts, recip_ok, tab, sb, w0, w1);
      }
      // LDS row rho = Y-row within the tile; 8-byte chunk ti stored at position ti ^ tj (= ti ^
      // (rho / CPL)) so that the 16 column groups of a wave hit distinct banks.
      const uint32_t rho = CPL * tj + c;
      *reinterpret_cast<uint2 *>(lds_codes + rho * (kColTokens / 2) + 8 * (ti ^ tj)) = make_uint2(w0, w1);
      lds_scales[rho * (kColTokens / 16) + ti] = static_cast<uint8_t>(sb);
    }
    const int64_t tK0 = K0, tR0 = R0;
    // the next tile's loads go out before this tile's output leaves LDS
    if (tile + gridDim.x < p.ntiles) {
      locate(tile + gridDim.x);
      load_patch<ESZ, CPL>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, valid);
    }
    __syncthreads();
    // codes: COLS rows x 128 B; 8 lanes per row, 16 B each
#pragma unroll
    for (int it = 0; it < (COLS * kColTokens / 2) / (16 * kThreads); ++it) {
      const uint32_t idx = threadIdx.x + kThreads * it;
      const uint32_t rho = idx >> 3, s = idx & 7u;
      const uint32_t sw = (rho / CPL) & 15u;
      const uint32_t p0 = (2 * s) ^ sw;
      uint4 val = *reinterpret_cast<const uint4 *>(lds_codes + rho * (kColTokens / 2) + 8 * (p0 & ~1u));
      if (p0 & 1u) val = make_uint4(val.z, val.w, val.x, val.y);
      const int64_t row = tR0 + rho;
      const int64_t k0 = tK0 + 32 * s;  // first token of this 16-byte segment
      if (row < p.R && k0 < p.K) {
        uint8_t *dst = p.data + row * (p.K / 2) + k0 / 2;
        if (ALIGNED) {
          *reinterpret_cast<uint4 *>(dst) = val;
        } else {
          *reinterpret_cast<uint2 *>(dst) = make_uint2(val.x, val.y);
          if (k0 + 16 < p.K) *reinterpret_cast<uint2 *>(dst + 8) = make_uint2(val.z, val.w);
        }
      }
    }
    if constexpr (!B2D) {
      if (threadIdx.x < COLS) {
        const uint32_t rho = threadIdx.x;
        const int64_t row = tR0 + rho;
        if (row < p.R) {
          uint8_t *dst = p.scales + row * KB + tK0 / 16;
          const uint8_t *srcs = lds_scales + rho * (kColTokens / 16);
          if (ALIGNED) {
            *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(srcs);
          } else {
            for (int q = 0; q < kColTokens / 16; ++q)
              if (tK0 / 16 + q < KB) dst[q] = srcs[q];
          }
        }
      }
    }
    __syncthreads();
  }
}

// Pass 1 of the column-wise Hadamard variants: the largest |H16 D u| / 4 over every 16-token block
// of every column, the values col_kernel's transform produces (the 1/4 taken once, quarter_bits).
// The order of the blocks does not matter for a maximum, so each wave takes strips of 16 tokens x
// (64 lanes x 16 bytes): lane l holds 16 bytes (8 bf16 / 4 f32 columns) of each of the strip's 16
// rows, and a row is read as 1 KiB contiguous per wave (col_kernel's lane layout reads 128-256 B
// pieces).  Consecutive strips of a token group go to consecutive waves.
template <int ESZ>
__global__ __launch_bounds__(kThreads) void col_amax_kernel(ColArgs p, FastDiv ns, uint32_t nunits) {  // ns: strips per group
  constexpr int CPL = 16 / ESZ;  // columns per lane
  enter_group(p, p.nparts);
  p.partial_out += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  uint32_t sflip[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) sflip[t] = ((p.sign_word >> t) & 1u) << 31;
  uint32_t mx = 0;
  for (uint32_t u = (blockIdx.x * kThreads + threadIdx.x) >> 6; u < nunits; u += nwaves) {
    const uint32_t g = fdiv(u, ns);
    const int64_t kk = 16 * static_cast<int64_t>(g);
    const int64_t rr = (static_cast<int64_t>(u - g * ns.d) * 64 + lane) * CPL;
    RawN<ESZ, CPL> v[16];
    load_patch<ESZ, CPL>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, rr < p.R);  // R % 8 == 0
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float y[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = rawn_elem_signed<ESZ, CPL>(v[t], c, sflip[t]);
      rht16_butterfly<false>(y);
      mx = max(mx, __float_as_uint(block_absmax(y)));
    }
  }
  write_partial(quarter_bits(mx), p.partial_out);
}

__global__ void zero_ts_kernel(float *ts, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) ts[i] = 0.0f;
}

// ---- host-side dispatch -------------------------------------------------------------------------------
uint32_t clamp_grid(uint64_t want, uint64_t cap) {
  if (want < 1) want = 1;
  return static_cast<uint32_t>(want < cap ? want : cap);
}

// Workgroups of kThreads threads of `kernel` that the current device holds at once (0 if unknown),
// cached per kernel and device.
uint32_t resident_groups(const void *kernel) {
  struct Entry {
    const void *k;
    int dev;
    uint32_t n;
  };
  static Entry cache[64];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  for (int i = 0; i < used; ++i)
    if (cache[i].k == kernel && cache[i].dev == dev) return cache[i].n;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kThreads, 0) != hipSuccess)
    return 0;
  const uint32_t n = static_cast<uint32_t>(cus) * static_cast<uint32_t>(per);
  if (used < 64) cache[used++] = Entry{kernel, dev, n};
  return n;
}

template <int ESZ>
hipError_t dispatch_quantize(const QuantArgs &a) {
  const bool colwise = (a.flags & 1u) != 0;
  const bool b2d = (a.flags & 2u) != 0;
  const bool sr = (a.flags & 4u) != 0;
  const bool fos = (a.flags & 8u) != 0;
  const bool search = (a.flags & 32u) != 0;
  const float ts_div = (a.flags & 16u) != 0 ? 1792.0f : 2688.0f;  // amax / (4 * 448) or / (6 * 448)
  const int mode = sr ? kSR : (fos ? kFourOverSix : (search ? kSearch : kRNE));
  const int64_t ldx_bytes = a.ldx * ESZ;
  const uint32_t key0 = static_cast<uint32_t>(a.seed), key1 = static_cast<uint32_t>(a.seed >> 32);
  const uint8_t *x = static_cast<const uint8_t *>(a.x);
  uint32_t nparts = 1, band_p = 0;
  const uint32_t G = static_cast<uint32_t>(a.groups);
  const GroupStrides gs{a.x_group_bytes, a.R * a.K / 2, b2d ? (a.R / 16) * (a.K / 16) : a.R * (a.K / 16)};

  // geometry of the pass-2 kernels (needed for the transform variants of pass 1 as well)
  RowArgs ra{};
  ColArgs ca8{}, ca4{};  // column-wise tiles of 256 tokens x 128 / 64 columns (8 / 4 per lane)
  if (!colwise) {
    ra = RowArgs{x, ldx_bytes, static_cast<uint32_t>(a.R * (a.K / 16)), make_fastdiv(static_cast<uint32_t>(a.K / 16)), a.K,
                 a.workspace, 0, a.workspace, a.data, a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out,
                 ts_div, gs};
  } else {
    const uint32_t ntk = static_cast<uint32_t>((a.K + kColTokens - 1) / kColTokens);
    auto col_args = [&](int64_t cols) {
      const uint32_t ntr = static_cast<uint32_t>((a.R + cols - 1) / cols);
      return ColArgs{x, ldx_bytes, a.K, a.R, ntr * ntk, make_fastdiv(ntr), a.workspace, 0, a.workspace, a.data,
                     a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out, ts_div, gs};
    };
    ca8 = col_args(128);
    ca4 = col_args(64);
  }

  // ---- pass 1
  if (!a.rht) {
    const uint64_t row_bytes = static_cast<uint64_t>(a.cols) * ESZ;
    const uint32_t cpr = static_cast<uint32_t>(row_bytes / 16);
    const uint64_t total = static_cast<uint64_t>(a.rows) * cpr;
    nparts = clamp_grid((total + 8 * kAmaxThreads - 1) / (8 * kAmaxThreads), kAmaxParts);
    AmaxArgs am{x, ldx_bytes, static_cast<uint32_t>(total), make_fastdiv(cpr > 0 ? cpr : 1),
                static_cast<uint32_t>(static_cast<int64_t>(row_bytes) == ldx_bytes), a.workspace, a.x_group_bytes, 0};
    if (b2d && !colwise && row_bytes % 1024 == 0 && row_bytes > 0) {
      // a 16-row band holds row_bytes 16-byte chunks, row_bytes / 1024 slabs; the relabelling is a
      // bijection when each grid step holds a multiple of 8 whole bands
      const uint64_t P = row_bytes / 1024;
      if (P <= 32 && (P & (P - 1)) == 0 && nparts % (8 * P) == 0) am.band_p = static_cast<uint32_t>(P);
    }
    band_p = am.band_p;
    hipLaunchKernelGGL(amax_kernel<ESZ>, dim3(nparts, G), dim3(kAmaxThreads), 0, a.stream, am);
  } else if (!colwise) {
    nparts = clamp_grid((ra.nblocks + 4 * kThreads - 1) / (4 * kThreads), kPass1Parts);
    hipLaunchKernelGGL((row1d_kernel<ESZ, kRNE, true, true>), dim3(nparts, G), dim3(kThreads), 0, a.stream, ra);
  } else {
    // one round of resident workgroups: a second, partial round would run at a fraction of the
    // machine's bandwidth
    const uint32_t nstrips = static_cast<uint32_t>((a.R + 64 * (16 / ESZ) - 1) / (64 * (16 / ESZ)));
    const uint32_t nunits = static_cast<uint32_t>(a.K / 16) * nstrips;
    const uint32_t res = resident_groups(reinterpret_cast<const void *>(&col_amax_kernel<ESZ>));
    nparts = clamp_grid((nunits + 3) / 4, res > 0 && res < kPass1Parts ? res : kPass1Parts);
    hipLaunchKernelGGL(col_amax_kernel<ESZ>, dim3(nparts, G), dim3(kThreads), 0, a.stream, ca4, make_fastdiv(nstrips), nunits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // ---- pass 2
  if (!colwise && !b2d) {
    ra.nparts = nparts;
    const uint32_t grid = clamp_grid((ra.nblocks + kThreads - 1) / kThreads, kPass2Grid);
    // pass 1 left each slab of 1024 16-byte chunks (amax_kernel) or of 256 blocks (the transform's
    // row1d pass 1) on XCD (slab index mod 8) when its grid is a multiple of 8: pass 2 then takes the
    // blocks in that XCD order, last-read slab first (measured faster; see BlockOrder)
    ra.slab = (grid % 8 == 0 && nparts % 8 == 0) ? (a.rht ? 256u : 1024u / ESZ) : 0u;
    const dim3 g(grid, G), blk(kThreads);
#define NVFP4_ROW(MODE_, RHT_) hipLaunchKernelGGL((row1d_kernel<ESZ, MODE_, RHT_, false>), g, blk, 0, a.stream, ra)
    if (a.rht) {
      if (mode == kSR)
        NVFP4_ROW(kSR, true);
      else if (mode == kFourOverSix)
        NVFP4_ROW(kFourOverSix, true);
      else if (mode == kSearch)
        NVFP4_ROW(kSearch, true);
      else
        NVFP4_ROW(kRNE, true);
    } else {
      if (mode == kSR)
        NVFP4_ROW(kSR, false);
      else if (mode == kFourOverSix)
        NVFP4_ROW(kFourOverSix, false);
      else if (mode == kSearch)
        NVFP4_ROW(kSearch, false);
      else
        NVFP4_ROW(kRNE, false);
    }
#undef NVFP4_ROW
  } else if (!colwise && b2d) {
    const uint32_t nseg = static_cast<uint32_t>((a.K + 511) / 512);
    Row2dArgs r2{x, ldx_bytes, static_cast<uint32_t>((a.R / 16) * nseg), make_fastdiv(nseg), a.K, a.workspace, nparts,
                 a.data, a.scales, a.ts, ts_div, gs, 0};
    const uint32_t grid = clamp_grid((r2.ntasks + 3) / 4, kPass2Grid2D);
    r2.affine = (band_p != 0 && grid % 8 == 0) ? 1u : 0u;
    if (fos)
      hipLaunchKernelGGL((row2d_kernel<ESZ, true>), dim3(grid, G), dim3(kThreads), 0, a.stream, r2);
    else
      hipLaunchKernelGGL((row2d_kernel<ESZ, false>), dim3(grid, G), dim3(kThreads), 0, a.stream, r2);
  } else {
    ca8.nparts = nparts;
    ca4.nparts = nparts;
    const bool aligned = (a.K % kColTokens) == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15u) == 0;
    const dim3 block(kThreads);
    // 1D blocks hold 4 columns per lane (fewer registers: more waves per SIMD, twice the tiles);
    // 16x16 tiles 8 (a lane pair is a tile).  Nearest-even runs one round of resident workgroups (a
    // few tiles each, the next one loading during the current one); the VALU-bound modes two rounds.
#define NVFP4_COL(MODE_, RHT_, B2D_)                                                                          \
  do {                                                                                                       \
    constexpr int CPL_ = B2D_ ? 8 : 4;                                                                       \
    const ColArgs &cc = CPL_ == 4 ? ca4 : ca8;                                                               \
    uint32_t cap_ = kPass2Grid;                                                                              \
    if (MODE_ == kRNE && CPL_ == 4) {                                                                        \
      const uint32_t res_ = resident_groups(                                                                 \
          reinterpret_cast<const void *>(&col_kernel<ESZ, MODE_, RHT_, B2D_, true, CPL_>));                  \
      if (res_ > 0 && res_ < cap_) cap_ = res_;                                                              \
    }                                                                                                        \
    const dim3 grid(clamp_grid(cc.ntiles, cap_), G);                                                         \
    if (aligned)                                                                                             \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, true, CPL_>), grid, block, 0, a.stream, cc); \
    else                                                                                                     \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, false, CPL_>), grid, block, 0, a.stream, cc); \
  } while (0)
    if (b2d && fos)
      NVFP4_COL(kFourOverSix, false, true);
    else if (b2d)
      NVFP4_COL(kRNE, false, true);
    else if (a.rht && mode == kSearch)
      NVFP4_COL(kSearch, true, false);
    else if (mode == kSearch)
      NVFP4_COL(kSearch, false, false);
    else if (a.rht && mode == kSR)
      NVFP4_COL(kSR, true, false);
    else if (a.rht && mode == kFourOverSix)
      NVFP4_COL(kFourOverSix, true, false);
    else if (a.rht)
      NVFP4_COL(kRNE, true, false);
    else if (mode == kSR)
      NVFP4_COL(kSR, false, false);
    else if (mode == kFourOverSix)
      NVFP4_COL(kFourOverSix, false, false);
    else
      NVFP4_COL(kRNE, false, false);
#undef NVFP4_COL
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a) {
  if (a.R == 0 || a.K == 0) {
    // empty tensor: ts = 0, nothing else to write (a kernel, not a memset, so that the call can be
    // captured in a graph)
    hipLaunchKernelGGL(zero_ts_kernel, dim3(1), dim3(64), 0, a.stream, a.ts, static_cast<uint32_t>(a.groups));
    return hipGetLastError();
  }
  return a.dtype == 1 ? dispatch_quantize<2>(a) : dispatch_quantize<4>(a);
}

namespace {
// The format's tensor scale for a tensor maximum: ts = RN(amax / 2688), as pass 1 computes it.
__global__ void scale_from_amax_kernel(const float *amax, float *ts) {
  if (threadIdx.x == 0) *ts = *amax / 2688.0f;
}
}  // namespace

hipError_t launch_scale_from_amax(const float *amax, float *ts, hipStream_t stream) {
  hipLaunchKernelGGL(scale_from_amax_kernel, dim3(1), dim3(64), 0, stream, amax, ts);
  return hipGetLastError();
}

}  // namespace nvfp4
