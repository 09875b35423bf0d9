// quantize.hip -- NVFP4 quantize kernels for gfx950 (HBM-bound).
//
// Two passes per tensor, both on the caller's stream:
//   pass 1  tensor amax: every workgroup writes the largest |y| it saw to workspace[blockIdx.x]
//           (plain tensors: amax_kernel; with the Hadamard transform the maximum is taken over the
//           transformed values, by the pass-2 kernels compiled with PASS1 = true);
//   pass 2  every wave reduces the partial maxima itself (no atomics, no zero-initialised memory),
//           derives ts = amax / 2688, and encodes its blocks: block amax -> E4M3 scale -> E2M1
//           codes (nearest-even, stochastic or Four-over-Six) -> packed nibbles.
// Layouts:
//   row1d_kernel   ROW mode, 1D blocks: one lane per 16-element block (32 B of bf16 in, 8 B out).
//   row2d_kernel   ROW mode, 16x16 tiles: a lane holds 16 rows x 8 columns; a lane pair is a tile.
//   col_kernel     COLWISE: a lane holds 16 tokens x 8 columns, i.e. one block of each of 8 rows of
//                  x^T; a 256-lane workgroup covers 256 tokens x 128 columns and transposes its
//                  packed output through LDS so that every row segment leaves as 128 contiguous
//                  bytes.
#include "nvfp4_device.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {

namespace {

constexpr uint32_t kThreads = 256;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---- loads ----------------------------------------------------------------------------------------
// 16 consecutive elements starting at p (32 B for bf16, 64 B for f32), widened to fp32.
template <int ESZ>
__device__ __forceinline__ void load16(const uint8_t *__restrict__ p, float (&y)[16]) {
  if constexpr (ESZ == 2) {
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint4 b = *reinterpret_cast<const uint4 *>(p + 16);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[2 * i] = bf16_lo(w[i]);
      y[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 a = *reinterpret_cast<const uint4 *>(p + 16 * i);
      y[4 * i] = __uint_as_float(a.x);
      y[4 * i + 1] = __uint_as_float(a.y);
      y[4 * i + 2] = __uint_as_float(a.z);
      y[4 * i + 3] = __uint_as_float(a.w);
    }
  }
}

// 8 consecutive elements at p (16 B bf16 / 32 B f32) kept raw.
template <int ESZ>
struct Raw8 {
  uint4 v[ESZ / 2];
};

template <int ESZ>
__device__ __forceinline__ Raw8<ESZ> load8(const uint8_t *__restrict__ p) {
  Raw8<ESZ> r;
#pragma unroll
  for (int i = 0; i < ESZ / 2; ++i) r.v[i] = *reinterpret_cast<const uint4 *>(p + 16 * i);
  return r;
}

template <int ESZ>
__device__ __forceinline__ float raw8_elem(const Raw8<ESZ> &r, int c) {
  if constexpr (ESZ == 2) {
    uint32_t w = (c >> 1) == 0 ? r.v[0].x : (c >> 1) == 1 ? r.v[0].y : (c >> 1) == 2 ? r.v[0].z : r.v[0].w;
    return (c & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    const uint4 &q = r.v[c >> 2];
    uint32_t w = (c & 3) == 0 ? q.x : (c & 3) == 1 ? q.y : (c & 3) == 2 ? q.z : q.w;
    return __uint_as_float(w);
  }
}

// ---- element codes --------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t sign_code(float y) { return (__float_as_uint(y) >> 28) & 8u; }

__device__ __forceinline__ uint32_t code_rne(float y, float e) {
  return e2m1_rne_index(fabsf(y) * e) | sign_code(y);
}

__device__ __forceinline__ uint32_t code_sr(float y, float e, uint32_t r16) {
  return e2m1_sr_index(fabsf(y) * e, r16) | sign_code(y);
}

// e == +inf (S * ts underflowed): nonzero elements saturate to 6, zeros stay zero.
__device__ __forceinline__ uint32_t code_degenerate(float y) {
  return (y == 0.0f ? 0u : 7u) | sign_code(y);
}

// Decode a code under scale S: RN(RN(q * S) * ts).
__device__ __forceinline__ float decode(uint32_t code, float S, float ts) {
  uint32_t idx = code & 7u;
  uint32_t qb = idx >= 2u ? (idx + 252u) << 22 : (idx == 1u ? 0x3F000000u : 0u);
  float q = __uint_as_float(qb | ((code & 8u) << 28));
  float p = q * S;
  return p * ts;
}

// Codes of one 16-element block under the given mode.  i0 = logical index of y[0] (a multiple of
// 16), used for the stochastic-rounding counter.
template <int MODE>
__device__ __forceinline__ void block_codes(const float (&y)[16], float e, uint64_t i0, uint32_t key0,
                                            uint32_t key1, uint32_t stream_id, uint32_t (&c)[16]) {
  if (__builtin_isinf(e)) {
#pragma unroll
    for (int t = 0; t < 16; ++t) c[t] = code_degenerate(y[t]);
  } else if constexpr (MODE == kSR) {
    uint64_t call = i0 >> 3;
    u32x4 r0 = philox4x32_10(static_cast<uint32_t>(call), static_cast<uint32_t>(call >> 32), stream_id, 0u, key0, key1);
    u32x4 r1 = philox4x32_10(static_cast<uint32_t>(call + 1), static_cast<uint32_t>((call + 1) >> 32), stream_id, 0u,
                             key0, key1);
#pragma unroll
    for (int t = 0; t < 8; ++t) c[t] = code_sr(y[t], e, r16_of(r0, t));
#pragma unroll
    for (int t = 0; t < 8; ++t) c[8 + t] = code_sr(y[8 + t], e, r16_of(r1, t));
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) c[t] = code_rne(y[t], e);
  }
}

__device__ __forceinline__ float block_sse(const float (&y)[16], const uint32_t (&c)[16], float S, float ts) {
  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    float diff = y[t] - decode(c[t], S, ts);
    acc = fmaf(diff, diff, acc);
  }
  return acc;
}

// Full encode of one 1D block: scale byte and two packed words (nibble t at bits 4t).
template <int MODE>
__device__ __forceinline__ void encode_block(const float (&y)[16], float ab, float ts, uint64_t i0, uint32_t key0,
                                             uint32_t key1, uint32_t stream_id, uint32_t &sbyte, uint32_t &w0,
                                             uint32_t &w1) {
  float S;
  sbyte = block_scale(ab, 6.0f, ts, S);
  uint32_t c[16];
  block_codes<MODE>(y, encode_factor(S, ts), i0, key0, key1, stream_id, c);
  if constexpr (MODE == kFourOverSix) {
    float acc6 = block_sse(y, c, S, ts);
    float S4;
    uint32_t sb4 = block_scale(ab, 4.0f, ts, S4);
    uint32_t c4[16];
    block_codes<kRNE>(y, encode_factor(S4, ts), i0, key0, key1, stream_id, c4);
    float acc4 = block_sse(y, c4, S4, ts);
    if (acc4 < acc6) {
      sbyte = sb4;
#pragma unroll
      for (int t = 0; t < 16; ++t) c[t] = c4[t];
    }
  }
  w0 = 0u;
  w1 = 0u;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    w0 |= c[t] << (4 * t);
    w1 |= c[8 + t] << (4 * t);
  }
}

__device__ __forceinline__ float block_absmax(const float (&y)[16]) {
  float ab = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) ab = fmaxf(ab, fabsf(y[t]));
  return ab;
}

// Workgroup max of one value per lane -> partial[blockIdx.x] (thread 0).
__device__ __forceinline__ void write_partial(uint32_t m, uint32_t *__restrict__ partial) {
  __shared__ uint32_t red[kThreads / 64];
  m = wave_max_u32(m);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (uint32_t w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
    partial[blockIdx.x] = r;
  }
}

// Every wave: tensor amax from the partials, ts = amax / 2688; block 0 publishes ts.
__device__ __forceinline__ float tensor_scale(const uint32_t *__restrict__ partial, uint32_t nparts,
                                              float *__restrict__ ts_out) {
  float A = tensor_amax(partial, nparts);
  float ts = A / 2688.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *ts_out = ts;
  return ts;
}

// ---- pass 1: plain tensor amax ----------------------------------------------------------------------
struct AmaxArgs {
  const uint8_t *x;
  int64_t ldx_bytes;
  uint32_t total_chunks;  // 16-byte chunks
  FastDiv cpr;            // chunks per row
  uint32_t flat;          // rows are contiguous (ldx == row length)
  uint32_t *partial;
};

template <int ESZ>
__device__ __forceinline__ void absmax_chunk(const uint4 &v, u16x2 &m2, uint32_t &m4) {
  if constexpr (ESZ == 2) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u16x2 a = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
      m2 = __builtin_elementwise_max(m2, a);
    }
  } else {
    m4 = max(m4, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
  }
}

template <int ESZ>
__global__ __launch_bounds__(kThreads) void amax_kernel(AmaxArgs p) {
  const uint32_t stride = gridDim.x * kThreads;
  u16x2 m2 = {0, 0};
  uint32_t m4 = 0;
  auto addr = [&](uint32_t c) -> const uint4 * {
    if (p.flat) return reinterpret_cast<const uint4 *>(p.x) + c;
    uint32_t r = fdiv(c, p.cpr);
    return reinterpret_cast<const uint4 *>(p.x + static_cast<int64_t>(r) * p.ldx_bytes +
                                           static_cast<int64_t>(c - r * p.cpr.d) * 16);
  };
  uint32_t c = blockIdx.x * kThreads + threadIdx.x;
  for (; c + 3 * stride < p.total_chunks; c += 4 * stride) {
    uint4 v0 = *addr(c), v1 = *addr(c + stride), v2 = *addr(c + 2 * stride), v3 = *addr(c + 3 * stride);
    absmax_chunk<ESZ>(v0, m2, m4);
    absmax_chunk<ESZ>(v1, m2, m4);
    absmax_chunk<ESZ>(v2, m2, m4);
    absmax_chunk<ESZ>(v3, m2, m4);
  }
  for (; c < p.total_chunks; c += stride) absmax_chunk<ESZ>(*addr(c), m2, m4);
  uint32_t m = ESZ == 2 ? (static_cast<uint32_t>(max(m2.x, m2.y)) << 16) : m4;
  write_partial(m, p.partial);
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
};

template <int ESZ, int MODE, bool RHT, bool PASS1>
__global__ __launch_bounds__(kThreads) void row1d_kernel(RowArgs p) {
  float ts = 0.0f;
  if constexpr (!PASS1) ts = tensor_scale(p.partial, p.nparts, p.ts_out);
  uint32_t mx = 0;
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < p.nblocks; b += stride) {
    const uint32_t r = fdiv(b, p.kb);
    const uint32_t kb = b - r * p.kb.d;
    float y[16];
    load16<ESZ>(p.x + static_cast<int64_t>(r) * p.ldx_bytes + static_cast<int64_t>(kb) * 16 * ESZ, y);
    if constexpr (RHT) rht16(y, p.sign_word);
    if constexpr (PASS1) {
      mx = max(mx, __float_as_uint(block_absmax(y)));
      continue;
    }
    const uint64_t i0 = static_cast<uint64_t>(r) * static_cast<uint64_t>(p.K) + 16u * kb;
    if constexpr (RHT) {
      if (p.rht_out) {
        float4 *o = reinterpret_cast<float4 *>(p.rht_out + i0);
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = make_float4(y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]);
      }
    }
    uint32_t sb, w0, w1;
    encode_block<MODE>(y, block_absmax(y), ts, i0, p.key0, p.key1, p.stream_id, sb, w0, w1);
    *reinterpret_cast<uint2 *>(p.data + (i0 >> 1)) = make_uint2(w0, w1);
    p.scales[i0 >> 4] = static_cast<uint8_t>(sb);
  }
  if constexpr (PASS1) write_partial(mx, p.partial_out);
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
};

template <int ESZ>
__global__ __launch_bounds__(kThreads) void row2d_kernel(Row2dArgs p) {
  const float ts = tensor_scale(p.partial, p.nparts, p.ts_out);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const int64_t KB = p.K / 16;
  for (uint32_t task = (blockIdx.x * kThreads + threadIdx.x) >> 6; task < p.ntasks; task += nwaves) {
    const uint32_t band = fdiv(task, p.nseg);
    const uint32_t seg = task - band * p.nseg.d;
    const int64_t r0 = static_cast<int64_t>(band) * 16;
    const int64_t c0 = static_cast<int64_t>(seg) * 512 + lane * 8;
    const bool valid = c0 < p.K;  // K % 16 == 0: both lanes of a tile agree
    Raw8<ESZ> v[16];
    float ab = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (valid) {
        v[t] = load8<ESZ>(p.x + (r0 + t) * p.ldx_bytes + c0 * ESZ);
      } else {
#pragma unroll
        for (int i = 0; i < ESZ / 2; ++i) v[t].v[i] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int c = 0; c < 8; ++c) ab = fmaxf(ab, fabsf(raw8_elem<ESZ>(v[t], c)));
    ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
    float S;
    const uint32_t sb = block_scale(ab, 6.0f, ts, S);
    const float e = encode_factor(S, ts);
    if (valid) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float yv = raw8_elem<ESZ>(v[t], c);
          uint32_t code = __builtin_isinf(e) ? code_degenerate(yv) : code_rne(yv, e);
          w |= code << (4 * c);
        }
        *reinterpret_cast<uint32_t *>(p.data + (r0 + t) * (p.K / 2) + c0 / 2) = w;
      }
      if ((lane & 1u) == 0) p.scales[(r0 / 16) * KB + c0 / 16] = static_cast<uint8_t>(sb);
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
};

constexpr int kColTokens = 256;  // per workgroup tile
constexpr int kColCols = 128;

template <int ESZ, int MODE, bool RHT, bool B2D, bool PASS1, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void col_kernel(ColArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[kColCols * (kColTokens / 2)];
  __shared__ __attribute__((aligned(16))) uint8_t lds_scales[kColCols * (kColTokens / 16)];
  float ts = 0.0f;
  if constexpr (!PASS1) ts = tensor_scale(p.partial, p.nparts, p.ts_out);
  const uint32_t ti = threadIdx.x >> 4;  // token group (16 tokens)
  const uint32_t tj = threadIdx.x & 15;  // column group (8 columns)
  const int64_t KB = p.K / 16;
  uint32_t mx = 0;
  for (uint32_t tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    const uint32_t tk = fdiv(tile, p.ntr);
    const uint32_t tr = tile - tk * p.ntr.d;
    const int64_t K0 = static_cast<int64_t>(tk) * kColTokens;
    const int64_t R0 = static_cast<int64_t>(tr) * kColCols;
    const int64_t kk = K0 + 16 * ti;
    const int64_t rr = R0 + 8 * tj;
    const bool valid = kk < p.K && rr < p.R;  // K % 16 == 0 and R % 8 == 0
    Raw8<ESZ> v[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (valid) {
        v[t] = load8<ESZ>(p.x + (kk + t) * p.ldx_bytes + rr * ESZ);
      } else {
#pragma unroll
        for (int i = 0; i < ESZ / 2; ++i) v[t].v[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if constexpr (PASS1) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float u[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) u[t] = raw8_elem<ESZ>(v[t], c);
        if constexpr (RHT) rht16(u, p.sign_word);
        mx = max(mx, __float_as_uint(block_absmax(u)));
      }
      continue;
    }
    float S2d = 0.0f, e2d = 0.0f;
    uint32_t sb2d = 0;
    if constexpr (B2D) {
      float ab = 0.0f;
#pragma unroll
      for (int t = 0; t < 16; ++t)
#pragma unroll
        for (int c = 0; c < 8; ++c) ab = fmaxf(ab, fabsf(raw8_elem<ESZ>(v[t], c)));
      ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
      sb2d = block_scale(ab, 6.0f, ts, S2d);
      e2d = encode_factor(S2d, ts);
      if (valid && (tj & 1u) == 0) p.scales[(rr / 16) * KB + kk / 16] = static_cast<uint8_t>(sb2d);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float u[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) u[t] = raw8_elem<ESZ>(v[t], c);
      if constexpr (RHT) rht16(u, p.sign_word);
      const uint64_t i0 = static_cast<uint64_t>(rr + c) * static_cast<uint64_t>(p.K) + static_cast<uint64_t>(kk);
      if constexpr (RHT) {
        if (p.rht_out && valid) {
          float4 *o = reinterpret_cast<float4 *>(p.rht_out + i0);
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = make_float4(u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]);
        }
      }
      uint32_t sb, w0, w1;
      if constexpr (B2D) {
        uint32_t cc[16];
        block_codes<kRNE>(u, e2d, i0, 0u, 0u, 0u, cc);
        w0 = 0u;
        w1 = 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          w0 |= cc[t] << (4 * t);
          w1 |= cc[8 + t] << (4 * t);
        }
        sb = sb2d;
      } else {
        encode_block<MODE>(u, block_absmax(u), ts, i0, p.key0, p.key1, p.stream_id, sb, w0, w1);
      }
      // LDS row rho = Y-row within the tile; 8-byte chunk ti stored at position ti ^ tj (= ti ^
      // (rho >> 3)) so that the 16 column groups of a wave hit distinct banks.
      const uint32_t rho = 8 * tj + c;
      *reinterpret_cast<uint2 *>(lds_codes + rho * (kColTokens / 2) + 8 * (ti ^ tj)) = make_uint2(w0, w1);
      lds_scales[rho * (kColTokens / 16) + ti] = static_cast<uint8_t>(sb);
    }
    __syncthreads();
    // codes: 128 rows x 128 B; 8 lanes per row, 16 B each
#pragma unroll
    for (int it = 0; it < (kColCols * kColTokens / 2) / (16 * kThreads); ++it) {
      const uint32_t idx = threadIdx.x + kThreads * it;
      const uint32_t rho = idx >> 3, s = idx & 7u;
      const uint32_t sw = (rho >> 3) & 15u;
      const uint32_t p0 = (2 * s) ^ sw;
      uint4 val = *reinterpret_cast<const uint4 *>(lds_codes + rho * (kColTokens / 2) + 8 * (p0 & ~1u));
      if (p0 & 1u) val = make_uint4(val.z, val.w, val.x, val.y);
      const int64_t row = R0 + rho;
      const int64_t k0 = K0 + 32 * s;  // first token of this 16-byte segment
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
      if (threadIdx.x < kColCols) {
        const uint32_t rho = threadIdx.x;
        const int64_t row = R0 + rho;
        if (row < p.R) {
          uint8_t *dst = p.scales + row * KB + K0 / 16;
          const uint8_t *src = lds_scales + rho * (kColTokens / 16);
          if (ALIGNED) {
            *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
          } else {
            for (int q = 0; q < kColTokens / 16; ++q)
              if (K0 / 16 + q < KB) dst[q] = src[q];
          }
        }
      }
    }
    __syncthreads();
  }
  if constexpr (PASS1) write_partial(mx, p.partial_out);
}

// ---- host-side dispatch -------------------------------------------------------------------------------
uint32_t clamp_grid(uint64_t want, uint64_t cap) {
  if (want < 1) want = 1;
  return static_cast<uint32_t>(want < cap ? want : cap);
}

template <int ESZ>
hipError_t dispatch_quantize(const QuantArgs &a) {
  const bool colwise = (a.flags & 1u) != 0;
  const bool b2d = (a.flags & 2u) != 0;
  const bool sr = (a.flags & 4u) != 0;
  const bool fos = (a.flags & 8u) != 0;
  const int mode = sr ? kSR : (fos ? kFourOverSix : kRNE);
  const int64_t ldx_bytes = a.ldx * ESZ;
  const uint32_t key0 = static_cast<uint32_t>(a.seed), key1 = static_cast<uint32_t>(a.seed >> 32);
  const uint8_t *x = static_cast<const uint8_t *>(a.x);
  uint32_t nparts = 1;

  // geometry of the pass-2 kernels (needed for the transform variants of pass 1 as well)
  RowArgs ra{};
  ColArgs ca{};
  uint32_t col_tiles = 0;
  if (!colwise) {
    ra = RowArgs{x, ldx_bytes, static_cast<uint32_t>(a.R * (a.K / 16)), make_fastdiv(static_cast<uint32_t>(a.K / 16)), a.K,
                 a.workspace, 0, a.workspace, a.data, a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out};
  } else {
    const uint32_t ntr = static_cast<uint32_t>((a.R + kColCols - 1) / kColCols);
    const uint32_t ntk = static_cast<uint32_t>((a.K + kColTokens - 1) / kColTokens);
    col_tiles = ntr * ntk;
    ca = ColArgs{x, ldx_bytes, a.K, a.R, col_tiles, make_fastdiv(ntr), a.workspace, 0, a.workspace, a.data,
                 a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out};
  }

  // ---- pass 1
  if (!a.rht) {
    const uint64_t row_bytes = static_cast<uint64_t>(a.cols) * ESZ;
    const uint32_t cpr = static_cast<uint32_t>(row_bytes / 16);
    const uint64_t total = static_cast<uint64_t>(a.rows) * cpr;
    nparts = clamp_grid((total + 4 * kThreads - 1) / (4 * kThreads), kMaxParts);
    AmaxArgs am{x, ldx_bytes, static_cast<uint32_t>(total), make_fastdiv(cpr > 0 ? cpr : 1),
                static_cast<uint32_t>(static_cast<int64_t>(row_bytes) == ldx_bytes), a.workspace};
    hipLaunchKernelGGL(amax_kernel<ESZ>, dim3(nparts), dim3(kThreads), 0, a.stream, am);
  } else if (!colwise) {
    nparts = clamp_grid((ra.nblocks + 4 * kThreads - 1) / (4 * kThreads), kMaxParts);
    hipLaunchKernelGGL((row1d_kernel<ESZ, kRNE, true, true>), dim3(nparts), dim3(kThreads), 0, a.stream, ra);
  } else {
    nparts = clamp_grid(col_tiles, kMaxParts);
    hipLaunchKernelGGL((col_kernel<ESZ, kRNE, true, false, true, false>), dim3(nparts), dim3(kThreads), 0, a.stream, ca);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // ---- pass 2
  if (!colwise && !b2d) {
    ra.nparts = nparts;
    const uint32_t grid = clamp_grid((ra.nblocks + kThreads - 1) / kThreads, 1u << 30);
    if (a.rht) {
      if (mode == kSR)
        hipLaunchKernelGGL((row1d_kernel<ESZ, kSR, true, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
      else if (mode == kFourOverSix)
        hipLaunchKernelGGL((row1d_kernel<ESZ, kFourOverSix, true, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
      else
        hipLaunchKernelGGL((row1d_kernel<ESZ, kRNE, true, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
    } else {
      if (mode == kSR)
        hipLaunchKernelGGL((row1d_kernel<ESZ, kSR, false, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
      else if (mode == kFourOverSix)
        hipLaunchKernelGGL((row1d_kernel<ESZ, kFourOverSix, false, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
      else
        hipLaunchKernelGGL((row1d_kernel<ESZ, kRNE, false, false>), dim3(grid), dim3(kThreads), 0, a.stream, ra);
    }
  } else if (!colwise && b2d) {
    const uint32_t nseg = static_cast<uint32_t>((a.K + 511) / 512);
    Row2dArgs r2{x, ldx_bytes, static_cast<uint32_t>((a.R / 16) * nseg), make_fastdiv(nseg), a.K, a.workspace, nparts,
                 a.data, a.scales, a.ts};
    const uint32_t grid = clamp_grid((r2.ntasks + 3) / 4, 1u << 30);
    hipLaunchKernelGGL(row2d_kernel<ESZ>, dim3(grid), dim3(kThreads), 0, a.stream, r2);
  } else {
    ca.nparts = nparts;
    const bool aligned = (a.K % kColTokens) == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15u) == 0;
    const dim3 grid(col_tiles), block(kThreads);
#define NVFP4_COL(MODE_, RHT_, B2D_)                                                                        \
  do {                                                                                                     \
    if (aligned)                                                                                           \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, false, true>), grid, block, 0, a.stream, ca); \
    else                                                                                                   \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, false, false>), grid, block, 0, a.stream, ca); \
  } while (0)
    if (b2d)
      NVFP4_COL(kRNE, false, true);
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

__global__ void zero_ts_kernel(float *ts) { *ts = 0.0f; }

}  // namespace

hipError_t launch_quantize(const QuantArgs &a) {
  if (a.R == 0 || a.K == 0) {
    // empty tensor: ts = 0, nothing else to write (a kernel, not a memset, so that the call can be
    // captured in a graph)
    hipLaunchKernelGGL(zero_ts_kernel, dim3(1), dim3(1), 0, a.stream, a.ts);
    return hipGetLastError();
  }
  return a.dtype == 1 ? dispatch_quantize<2>(a) : dispatch_quantize<4>(a);
}

}  // namespace nvfp4
