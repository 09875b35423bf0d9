// quantize.hip -- NVFP4 quantize kernels for gfx950 (HBM-bound).
//
// Two passes per tensor, both on the caller's stream:
//   pass 1  tensor amax: every workgroup writes the largest |y| it saw to workspace[blockIdx.x]
//           (plain tensors: amax_kernel; with the Hadamard transform the maximum is taken over the
//           transformed values, by the pass-2 kernels compiled with PASS1 = true);
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
constexpr uint32_t kPass1Parts = 1024; // pass-1 workgroups at most (<= kMaxParts): the partial maxima
                                       // every pass-2 wave reduces
constexpr uint32_t kAmaxThreads = 1024; // amax_kernel workgroup: one per CU, 16 waves
constexpr uint32_t kAmaxParts = 256;
constexpr uint32_t kPass2Grid = 2048;  // persistent pass-2 workgroups (8 per CU)
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
__device__ __forceinline__ uint32_t code_sr(float y, float e, uint32_t r16) {
  return e2m1_sr_index(fabsf(y) * e, r16) | sign_code(y);
}

// Decoded error terms of one byte of packed codes (two elements, low nibble first) under scale S:
// the decoded value is RN(RN(q * S) * ts), where q * S is exact (q has at most two significant bits,
// S four, and the product stays normal).  v_cvt_scalef32_pk_f32_fp4 with scale 1.0 returns the two
// E2M1 values q exactly, so each element costs half a conversion and two multiplies.
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
  if (__builtin_isinf(e)) {
    w0 = 0u;
    w1 = 0u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      w0 |= code_degenerate(y[t]) << (4 * t);
      w1 |= code_degenerate(y[8 + t]) << (4 * t);
    }
  } else if constexpr (MODE == kSR) {
    const uint64_t call = i0 >> 3;
    const u32x4 r0 = philox4x32_10(static_cast<uint32_t>(call), static_cast<uint32_t>(call >> 32), stream_id, 0u,
                                   key0, key1);
    const u32x4 r1 = philox4x32_10(static_cast<uint32_t>(call + 1), static_cast<uint32_t>((call + 1) >> 32),
                                   stream_id, 0u, key0, key1);
    w0 = 0u;
    w1 = 0u;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      w0 |= code_sr(y[t], e, r16_of(r0, t)) << (4 * t);
      w1 |= code_sr(y[8 + t], e, r16_of(r1, t)) << (4 * t);
    }
  } else {
    w0 = pack8_rne(y, e);
    w1 = pack8_rne(y + 8, e);
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
  constexpr int U = 8;  // loads in flight per lane
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
  uint32_t c = blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; c + (U - 1) * stride < p.total_chunks; c += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *addr(c + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) absmax_chunk<ESZ>(v[u], m2, m4);
  }
  for (; c < p.total_chunks; c += stride) absmax_chunk<ESZ>(*addr(c), m2, m4);
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
};

template <int ESZ, int MODE, bool RHT, bool PASS1>
__global__ __launch_bounds__(kThreads) void row1d_kernel(RowArgs p) {
  enter_group(p, p.nparts);
  p.partial_out += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  p.stream_id += blockIdx.y;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  auto src = [&](uint32_t blk) {
    const uint32_t r = fdiv(blk, p.kb);
    return p.x + static_cast<int64_t>(r) * p.ldx_bytes + static_cast<int64_t>(blk - r * p.kb.d) * 16 * ESZ;
  };
  Raw16<ESZ> cur, nxt;
  if (b < p.nblocks) cur = load_raw16<ESZ>(src(b));
  float ts = 0.0f;
  if constexpr (!PASS1) ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  uint32_t mx = 0;
  while (b < p.nblocks) {
    const uint32_t bn = b + stride;
    if (bn < p.nblocks) nxt = load_raw16<ESZ>(src(bn));
    float y[16];
    unpack16<ESZ>(cur, y);
    if constexpr (RHT) rht16(y, p.sign_word);
    if constexpr (PASS1) {
      mx = max(mx, __float_as_uint(block_absmax(y)));
    } else {
      const uint32_t r = fdiv(b, p.kb);
      const uint64_t i0 = static_cast<uint64_t>(r) * static_cast<uint64_t>(p.K) + 16u * (b - r * p.kb.d);
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
    cur = nxt;
    b = bn;
  }
  if constexpr (PASS1) write_partial(mx, p.partial_out);
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

// fp32 squared error of 8 values against their codes w under scale S, accumulated into acc with fma
// in order.
__device__ __forceinline__ float sse8(const float (&yv)[8], uint32_t w, float S, float ts, float acc) {
  acc = sse_pair<0>(w, yv[0], yv[1], S, ts, acc);
  acc = sse_pair<1>(w, yv[2], yv[3], S, ts, acc);
  acc = sse_pair<2>(w, yv[4], yv[5], S, ts, acc);
  return sse_pair<3>(w, yv[6], yv[7], S, ts, acc);
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
};

template <int ESZ>
__device__ __forceinline__ void load_patch(Raw8<ESZ> (&v)[16], const uint8_t *__restrict__ base, int64_t ld_bytes,
                                           bool valid) {
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    if (valid) {
      v[t] = load8<ESZ>(base + t * ld_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < ESZ / 2; ++i) v[t].v[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

// Four-over-Six tile error for the lane pair of a 16x16 tile (even lane: columns 0-7, odd lane:
// columns 8-15, each 16 rows): quadrant sums in row-major order, (TL + TR) + (BL + BR).
template <int ESZ>
__device__ __forceinline__ float tile_sse_rows(const Raw8<ESZ> (&v)[16], float e, float S, float ts) {
  float top = 0.0f, bottom = 0.0f;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    float yv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) yv[c] = raw8_elem<ESZ>(v[t], c);
    const uint32_t w = codes8(yv, e);
    if (t < 8)
      top = sse8(yv, w, S, ts, top);
    else
      bottom = sse8(yv, w, S, ts, bottom);
  }
  const float top_o = __shfl_xor(top, 1, 64), bottom_o = __shfl_xor(bottom, 1, 64);
  return (top + top_o) + (bottom + bottom_o);
}

template <int ESZ, bool FOS>
__global__ __launch_bounds__(kThreads) void row2d_kernel(Row2dArgs p) {
  enter_group(p, p.nparts);
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t nwaves = gridDim.x * (kThreads / 64);
  const int64_t KB = p.K / 16;
  uint32_t task = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  Raw8<ESZ> v[16];
  auto start = [&](uint32_t tk, int64_t &r0, int64_t &c0) {
    const uint32_t band = fdiv(tk, p.nseg);
    r0 = static_cast<int64_t>(band) * 16;
    c0 = static_cast<int64_t>(tk - band * p.nseg.d) * 512 + lane * 8;
  };
  int64_t r0 = 0, c0 = 0;
  if (task < p.ntasks) {
    start(task, r0, c0);
    load_patch<ESZ>(v, p.x + r0 * p.ldx_bytes + c0 * ESZ, p.ldx_bytes, c0 < p.K);
  }
  const float ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  while (task < p.ntasks) {
    const bool valid = c0 < p.K;  // K % 16 == 0: both lanes of a tile agree
    float ab = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t)
#pragma unroll
      for (int c = 0; c < 8; ++c) ab = fmaxf(ab, fabsf(raw8_elem<ESZ>(v[t], c)));
    ab = fmaxf(ab, __shfl_xor(ab, 1, 64));
    float S;
    uint32_t sb = block_scale(ab, 6.0f, ts, S);
    float e = encode_factor(S, ts);
    if constexpr (FOS) {
      // Four-over-Six on the tile: target 4 only if its tile error is strictly lower
      const float sse6 = tile_sse_rows<ESZ>(v, e, S, ts);
      float S4;
      const uint32_t sb4 = block_scale(ab, 4.0f, ts, S4);
      const float e4 = encode_factor(S4, ts);
      const float sse4 = tile_sse_rows<ESZ>(v, e4, S4, ts);
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
    task += nwaves;
    if (task < p.ntasks) {
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
constexpr int kColCols = 128;

template <int ESZ, int MODE, bool RHT, bool B2D, bool PASS1, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void col_kernel(ColArgs p) {
  enter_group(p, p.nparts);
  p.partial_out += static_cast<int64_t>(blockIdx.y) * gridDim.x;
  p.stream_id += blockIdx.y;
  __shared__ __attribute__((aligned(16))) uint8_t lds_codes[kColCols * (kColTokens / 2)];
  __shared__ __attribute__((aligned(16))) uint8_t lds_scales[kColCols * (kColTokens / 16)];
  const uint32_t ti = threadIdx.x >> 4;  // token group (16 tokens)
  const uint32_t tj = threadIdx.x & 15;  // column group (8 columns)
  const int64_t KB = p.K / 16;
  uint32_t mx = 0;
  Raw8<ESZ> v[16];
  int64_t K0 = 0, R0 = 0, kk = 0, rr = 0;
  bool valid = false;
  auto locate = [&](uint32_t tile) {
    const uint32_t tk = fdiv(tile, p.ntr);
    K0 = static_cast<int64_t>(tk) * kColTokens;
    R0 = static_cast<int64_t>(tile - tk * p.ntr.d) * kColCols;
    kk = K0 + 16 * ti;
    rr = R0 + 8 * tj;
    valid = kk < p.K && rr < p.R;  // K % 16 == 0 and R % 8 == 0
  };
  uint32_t tile = blockIdx.x;
  if (tile < p.ntiles) {
    locate(tile);
    load_patch<ESZ>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, valid);
  }
  float ts = 0.0f;
  if constexpr (!PASS1) ts = tensor_scale(p.partial, p.nparts, p.ts_out, p.ts_div);
  for (; tile < p.ntiles; tile += gridDim.x) {
    if constexpr (PASS1) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float u[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) u[t] = raw8_elem<ESZ>(v[t], c);
        if constexpr (RHT) rht16(u, p.sign_word);
        mx = max(mx, __float_as_uint(block_absmax(u)));
      }
      if (tile + gridDim.x < p.ntiles) {
        locate(tile + gridDim.x);
        load_patch<ESZ>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, valid);
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
      if constexpr (MODE == kFourOverSix) {
        // Four-over-Six on the tile: this lane holds 8 rows (top or bottom half of the tile) of all
        // 16 columns; quadrant sums in row-major order, (TL + TR) + (BL + BR)
        auto tile_sse = [&](float e, float S) {
          float left = 0.0f, right = 0.0f;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float a[8], b[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              a[t] = raw8_elem<ESZ>(v[t], c);
              b[t] = raw8_elem<ESZ>(v[8 + t], c);
            }
            left = sse8(a, codes8(a, e), S, ts, left);
            right = sse8(b, codes8(b, e), S, ts, right);
          }
          const float half = left + right;
          return half + __shfl_xor(half, 1, 64);
        };
        const float sse6 = tile_sse(e2d, S2d);
        float S4;
        const uint32_t sb4 = block_scale(ab, 4.0f, ts, S4);
        const float e4 = encode_factor(S4, ts);
        const float sse4 = tile_sse(e4, S4);
        if (sse4 < sse6) {
          sb2d = sb4;
          S2d = S4;
          e2d = e4;
        }
      }
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
        block_words<kRNE>(u, e2d, i0, 0u, 0u, 0u, w0, w1);
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
    const int64_t tK0 = K0, tR0 = R0;
    // the next tile's loads go out before this tile's output leaves LDS
    if (tile + gridDim.x < p.ntiles) {
      locate(tile + gridDim.x);
      load_patch<ESZ>(v, p.x + kk * p.ldx_bytes + rr * ESZ, p.ldx_bytes, valid);
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
      if (threadIdx.x < kColCols) {
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
  if constexpr (PASS1) write_partial(mx, p.partial_out);
}

__global__ void zero_ts_kernel(float *ts, uint32_t n) {
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) ts[i] = 0.0f;
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
  const bool search = (a.flags & 32u) != 0;
  const float ts_div = (a.flags & 16u) != 0 ? 1792.0f : 2688.0f;  // amax / (4 * 448) or / (6 * 448)
  const int mode = sr ? kSR : (fos ? kFourOverSix : (search ? kSearch : kRNE));
  const int64_t ldx_bytes = a.ldx * ESZ;
  const uint32_t key0 = static_cast<uint32_t>(a.seed), key1 = static_cast<uint32_t>(a.seed >> 32);
  const uint8_t *x = static_cast<const uint8_t *>(a.x);
  uint32_t nparts = 1;
  const uint32_t G = static_cast<uint32_t>(a.groups);
  const GroupStrides gs{a.x_group_bytes, a.R * a.K / 2, b2d ? (a.R / 16) * (a.K / 16) : a.R * (a.K / 16)};

  // geometry of the pass-2 kernels (needed for the transform variants of pass 1 as well)
  RowArgs ra{};
  ColArgs ca{};
  uint32_t col_tiles = 0;
  if (!colwise) {
    ra = RowArgs{x, ldx_bytes, static_cast<uint32_t>(a.R * (a.K / 16)), make_fastdiv(static_cast<uint32_t>(a.K / 16)), a.K,
                 a.workspace, 0, a.workspace, a.data, a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out,
                 ts_div, gs};
  } else {
    const uint32_t ntr = static_cast<uint32_t>((a.R + kColCols - 1) / kColCols);
    const uint32_t ntk = static_cast<uint32_t>((a.K + kColTokens - 1) / kColTokens);
    col_tiles = ntr * ntk;
    ca = ColArgs{x, ldx_bytes, a.K, a.R, col_tiles, make_fastdiv(ntr), a.workspace, 0, a.workspace, a.data,
                 a.scales, a.ts, key0, key1, a.stream_id, a.sign_word, a.rht_out, ts_div, gs};
  }

  // ---- pass 1
  if (!a.rht) {
    const uint64_t row_bytes = static_cast<uint64_t>(a.cols) * ESZ;
    const uint32_t cpr = static_cast<uint32_t>(row_bytes / 16);
    const uint64_t total = static_cast<uint64_t>(a.rows) * cpr;
    nparts = clamp_grid((total + 8 * kAmaxThreads - 1) / (8 * kAmaxThreads), kAmaxParts);
    AmaxArgs am{x, ldx_bytes, static_cast<uint32_t>(total), make_fastdiv(cpr > 0 ? cpr : 1),
                static_cast<uint32_t>(static_cast<int64_t>(row_bytes) == ldx_bytes), a.workspace, a.x_group_bytes};
    hipLaunchKernelGGL(amax_kernel<ESZ>, dim3(nparts, G), dim3(kAmaxThreads), 0, a.stream, am);
  } else if (!colwise) {
    nparts = clamp_grid((ra.nblocks + 4 * kThreads - 1) / (4 * kThreads), kPass1Parts);
    hipLaunchKernelGGL((row1d_kernel<ESZ, kRNE, true, true>), dim3(nparts, G), dim3(kThreads), 0, a.stream, ra);
  } else {
    nparts = clamp_grid(col_tiles, kPass1Parts);
    hipLaunchKernelGGL((col_kernel<ESZ, kRNE, true, false, true, false>), dim3(nparts, G), dim3(kThreads), 0, a.stream, ca);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  // ---- pass 2
  if (!colwise && !b2d) {
    ra.nparts = nparts;
    const uint32_t grid = clamp_grid((ra.nblocks + kThreads - 1) / kThreads, kPass2Grid);
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
                 a.data, a.scales, a.ts, ts_div, gs};
    const uint32_t grid = clamp_grid((r2.ntasks + 3) / 4, kPass2Grid);
    if (fos)
      hipLaunchKernelGGL((row2d_kernel<ESZ, true>), dim3(grid, G), dim3(kThreads), 0, a.stream, r2);
    else
      hipLaunchKernelGGL((row2d_kernel<ESZ, false>), dim3(grid, G), dim3(kThreads), 0, a.stream, r2);
  } else {
    ca.nparts = nparts;
    const bool aligned = (a.K % kColTokens) == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15u) == 0;
    const dim3 grid(clamp_grid(col_tiles, kPass2Grid), G), block(kThreads);
#define NVFP4_COL(MODE_, RHT_, B2D_)                                                                        \
  do {                                                                                                     \
    if (aligned)                                                                                           \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, false, true>), grid, block, 0, a.stream, ca); \
    else                                                                                                   \
      hipLaunchKernelGGL((col_kernel<ESZ, MODE_, RHT_, B2D_, false, false>), grid, block, 0, a.stream, ca); \
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
