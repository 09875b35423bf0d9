/*
 * nvfp4_oracle.cpp -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see nvfp4_oracle.h).
 *
 * Written for readability, not speed: tables are enumerated, the logical matrix Y is
 * materialised, and every step runs in the order the format reading fixes.  Build with
 *   g++ -O2 -std=c++17 -ffp-contract=off -fPIC -shared   (no -ffast-math)
 * so that no a*b+c is silently fused and every float operation is one IEEE binary32 operation.
 */
#include "nvfp4_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

namespace {

/* E2M1 magnitudes, indexed by the 3-bit magnitude field (2 exponent bits, bias 1, 1 mantissa bit):
 * the grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
const float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float widen_bf16(uint16_t h) {
  uint32_t b = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

/* Run fn(lo, hi) over [0, n) split into nthreads contiguous ranges (each a multiple of `grain`). */
void parallel_ranges(int64_t n, int64_t grain, int nthreads,
                     const std::function<void(int64_t, int64_t)> &fn) {
  if (nthreads <= 1 || n <= grain) {
    fn(0, n);
    return;
  }
  int64_t units = (n + grain - 1) / grain;
  int64_t per = (units + nthreads - 1) / nthreads;
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = static_cast<int64_t>(t) * per * grain;
    int64_t hi = std::min(n, lo + per * grain);
    if (lo >= hi) break;
    pool.emplace_back(fn, lo, hi);
  }
  for (auto &th : pool) th.join();
}

/* Block scale for target T (6, or 4 under Four-over-Six):
 * ts == 0 -> 0; else s = RN(RN(a_b / T) / ts), clamped to 448, then E4M3 round-to-nearest-even. */
uint8_t block_scale_byte(float a_b, float T, float ts) {
  if (ts == 0.0f) return 0;
  float q = a_b / T;
  float s = q / ts;
  if (!(s <= 448.0f)) s = 448.0f; /* s > 448 (or +inf after overflow) clamps to the E4M3 max */
  return static_cast<uint8_t>(or_e4m3_rne(s));
}

/* Lower grid neighbour index of v in [0, 6): the largest i with kE2M1[i] <= v. */
int grid_floor_index(float v) {
  int i = 0;
  while (i < 7 && kE2M1[i + 1] <= v) ++i;
  return i;
}

struct QuantCtx {
  int64_t R, K;
  uint32_t flags;
  uint64_t seed;
  uint32_t stream_id;
  float ts;
};

/* Sum of the n x n block at (r, c) of a 16x16 array of squared errors, over the quad tree: the
 * block splits into four n/2 x n/2 blocks, summed as (top-left + bottom-right) + (top-right +
 * bottom-left), down to single elements.  Transposing the tile maps the two diagonal blocks
 * onto themselves and swaps the two off-diagonal ones, so (float addition being commutative)
 * the tile and its transpose give the same sum. */
float quad_sum(const float *sq, int r, int c, int n) {
  if (n == 1) return sq[r * 16 + c];
  const int h = n / 2;
  float diag = quad_sum(sq, r, c, h) + quad_sum(sq, r + h, c + h, h);
  float off = quad_sum(sq, r, c + h, h) + quad_sum(sq, r + h, c, h);
  return diag + off;
}

/* Encode one element y of Y at (r, k) under scale byte sb.  Returns the 4-bit code. */
uint8_t encode_element(const QuantCtx &c, float y, uint8_t sb, int64_t r, int64_t k) {
  float S = or_e4m3_value(sb);
  int idx = 0;
  if (S != 0.0f && y != 0.0f) {
    float d = S * c.ts;
    float e = 1.0f / d;
    float v = std::fabs(y) * e;
    if (c.flags & OR_SR) {
      if (v >= 6.0f) {
        idx = 7;
      } else {
        int i = grid_floor_index(v);
        float lo = kE2M1[i], hi = kE2M1[i + 1];
        float f = (v - lo) / (hi - lo); /* exact: Sterbenz subtraction, power-of-two divisor */
        uint64_t el = static_cast<uint64_t>(r) * static_cast<uint64_t>(c.K) + static_cast<uint64_t>(k);
        uint64_t call = el >> 3;
        uint32_t ctr[4] = {static_cast<uint32_t>(call), static_cast<uint32_t>(call >> 32), c.stream_id, 0u};
        uint32_t key[2] = {static_cast<uint32_t>(c.seed), static_cast<uint32_t>(c.seed >> 32)};
        uint32_t w[4];
        or_philox4x32_10(ctr, key, w);
        uint32_t r16 = (w[(el & 7) >> 1] >> (16 * (el & 1))) & 0xFFFFu;
        bool up = static_cast<float>(r16) < f * 65536.0f;
        idx = up ? i + 1 : i;
      }
    } else {
      idx = or_e2m1_rne_index(v);
    }
  }
  return static_cast<uint8_t>((std::signbit(y) ? 8 : 0) | idx);
}

/* Dequantized value of a code under scale byte sb: RN(RN(q * S) * ts). */
float decode_element(uint8_t code, uint8_t sb, float ts) {
  float q = or_e2m1_value(code & 15);
  float S = or_e4m3_value(sb);
  float p = q * S;
  return p * ts;
}

} /* namespace */

extern "C" {

float or_e2m1_value(int code) {
  float m = kE2M1[code & 7];
  return (code & 8) ? -m : m;
}

int or_e2m1_rne_index(float v) {
  /* Enumerate the grid, keep the nearest; on an exact tie keep the even index (its mantissa
   * bit is 0).  Distances are formed in binary64, exact for every v near a grid midpoint. */
  if (!(v >= 0.0f)) return 0;
  if (v >= 6.0f) return 7; /* saturate: 6 is the largest grid value (also for +inf) */
  int best = 0;
  double bestd = std::fabs(static_cast<double>(v) - kE2M1[0]);
  for (int i = 1; i < 8; ++i) {
    double d = std::fabs(static_cast<double>(v) - kE2M1[i]);
    if (d < bestd || (d == bestd && (i % 2) == 0)) {
      best = i;
      bestd = d;
    }
  }
  return best;
}

float or_e4m3_value(int byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  float v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = std::ldexp(static_cast<float>(m), -9); /* subnormal: m * 2^-9 */
  else
    v = std::ldexp(static_cast<float>(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

int or_e4m3_rne(float s) {
  /* nearest of the 127 non-negative finite E4M3FN values 0x00..0x7E; ties to even byte */
  if (!(s > 0.0f)) return 0;
  if (s >= 448.0f) return 0x7E;
  int best = 0;
  double bestd = std::fabs(static_cast<double>(s));
  for (int b = 1; b <= 0x7E; ++b) {
    double d = std::fabs(static_cast<double>(s) - static_cast<double>(or_e4m3_value(b)));
    if (d < bestd || (d == bestd && (b % 2) == 0)) {
      best = b;
      bestd = d;
    }
  }
  return best;
}

void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  /* Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
   * 1, 2, 3", SC 2011): each round multiplies words 0 and 2 by the two round multipliers, mixes
   * the high halves with words 1/3 and the key, and the key is bumped by the Weyl constants. */
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t p0 = static_cast<uint64_t>(M0) * x0;
    uint64_t p1 = static_cast<uint64_t>(M1) * x2;
    uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

uint32_t or_rht_sign_word(uint64_t sign_seed) {
  uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  uint32_t key[2] = {static_cast<uint32_t>(sign_seed), static_cast<uint32_t>(sign_seed >> 32)};
  uint32_t w[4];
  or_philox4x32_10(ctr, key, w);
  return w[0] & 0xFFFFu;
}

void or_rht16(float u[16], uint32_t sign_word) {
  /* (1/4) H16 D u: D = diag of the seeded signs, H16 the Sylvester Hadamard matrix
   * H[i][j] = (-1)^popcount(i & j), applied as the radix-2 butterfly with strides 1, 2, 4, 8. */
  for (int t = 0; t < 16; ++t)
    if ((sign_word >> t) & 1u) u[t] = -u[t];
  for (int h = 1; h < 16; h *= 2) {
    for (int i = 0; i < 16; i += 2 * h) {
      for (int m = i; m < i + h; ++m) {
        float a = u[m];
        float b = u[m + h];
        u[m] = a + b;
        u[m + h] = a - b;
      }
    }
  }
  for (int t = 0; t < 16; ++t) u[t] = u[t] * 0.25f;
}

void or_e2m1_rne_array(const float *v, int64_t n, uint8_t *idx) {
  for (int64_t i = 0; i < n; ++i) idx[i] = static_cast<uint8_t>(or_e2m1_rne_index(v[i]));
}

void or_e4m3_rne_array(const float *s, int64_t n, uint8_t *bytes) {
  for (int64_t i = 0; i < n; ++i) bytes[i] = static_cast<uint8_t>(or_e4m3_rne(s[i]));
}

void or_philox_array(const uint32_t *ctr4, const uint32_t *key2, int64_t n, uint32_t *out4) {
  for (int64_t i = 0; i < n; ++i) or_philox4x32_10(ctr4 + 4 * i, key2 + 2 * i, out4 + 4 * i);
}

void or_rht16_array(float *u, int64_t nchunks, uint32_t sign_word) {
  for (int64_t i = 0; i < nchunks; ++i) or_rht16(u + 16 * i, sign_word);
}

int or_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, uint32_t flags,
                uint64_t seed, uint32_t stream_id, int use_rht, uint64_t sign_seed,
                uint8_t *data, uint8_t *scales, float *ts_out, float *rht_out, double *sse2,
                int nthreads) {
  const bool colwise = (flags & OR_COLWISE) != 0;
  const bool block2d = (flags & OR_BLOCK2D) != 0;
  const bool sr = (flags & OR_SR) != 0;
  const bool fos = (flags & OR_FOUR_OVER_SIX) != 0;
  const bool search = (flags & OR_SCALE_SEARCH) != 0;
  const bool ts_four = (flags & OR_TS_FOR_FOUR) != 0;
  if (rows < 0 || cols < 0 || ldx < cols) return 2;
  const int64_t R = colwise ? cols : rows;
  const int64_t K = colwise ? rows : cols;
  if (K % 16 != 0) return 2;
  if (block2d && R % 16 != 0) return 2;
  if ((sr && (fos || search)) || (sr && block2d) || (fos && search) || (search && block2d) ||
      (use_rht && block2d))
    return 4;

  /* Y[r][k] materialised in fp32 (bf16 widened exactly). */
  std::vector<float> Y(static_cast<size_t>(R * K));
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      int64_t src = colwise ? (k * ldx + r) : (r * ldx + k);
      float v = (dtype == OR_DT_BF16) ? widen_bf16(static_cast<const uint16_t *>(x)[src])
                                      : static_cast<const float *>(x)[src];
      Y[static_cast<size_t>(r * K + k)] = v;
    }
  }

  /* Optional 16x16 RHT on every 16-chunk of each row of Y. */
  if (use_rht) {
    uint32_t sw = or_rht_sign_word(sign_seed);
    parallel_ranges(R, 1, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t r = lo; r < hi; ++r)
        for (int64_t j = 0; j < K / 16; ++j) or_rht16(&Y[static_cast<size_t>(r * K + 16 * j)], sw);
    });
    if (rht_out) std::memcpy(rht_out, Y.data(), sizeof(float) * static_cast<size_t>(R * K));
  }

  /* Tensor amax and FP32 tensor scale ts = amax / (6 * 448). */
  std::vector<float> part(static_cast<size_t>(std::max(1, nthreads)), 0.0f);
  {
    int64_t per = (R + std::max(1, nthreads) - 1) / std::max(1, nthreads);
    std::vector<std::thread> pool;
    for (int t = 0; t < std::max(1, nthreads); ++t) {
      int64_t lo = t * per, hi = std::min(R, lo + per);
      if (lo >= hi) break;
      pool.emplace_back([&, t, lo, hi]() {
        float m = 0.0f;
        for (int64_t i = lo * K; i < hi * K; ++i) m = std::max(m, std::fabs(Y[static_cast<size_t>(i)]));
        part[static_cast<size_t>(t)] = m;
      });
    }
    for (auto &th : pool) th.join();
  }
  float A = 0.0f;
  for (float m : part) A = std::max(A, m);
  const float ts = ts_four ? A / 1792.0f : A / 2688.0f;
  *ts_out = ts;

  QuantCtx c{R, K, flags, seed, stream_id, ts};
  const int64_t KB = K / 16;
  std::vector<double> sse_chosen(static_cast<size_t>(R), 0.0), sse_plain(static_cast<size_t>(R), 0.0);

  auto store_code = [&](int64_t r, int64_t k, uint8_t code) {
    uint8_t &byte = data[r * (K / 2) + k / 2];
    if (k % 2 == 0)
      byte = static_cast<uint8_t>((byte & 0xF0) | code);
    else
      byte = static_cast<uint8_t>((byte & 0x0F) | (code << 4));
  };

  if (block2d) {
    parallel_ranges(R, 16, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t r0 = lo; r0 < hi; r0 += 16) {
        for (int64_t kb = 0; kb < KB; ++kb) {
          float ab = 0.0f;
          for (int64_t r = r0; r < r0 + 16; ++r)
            for (int64_t t = 0; t < 16; ++t)
              ab = std::max(ab, std::fabs(Y[static_cast<size_t>(r * K + 16 * kb + t)]));
          uint8_t sb = block_scale_byte(ab, 6.0f, ts);
          if (fos) {
            /* Four-over-Six on the tile: the same choice as for a 1D block, with the tile SSE
             * the quad-tree sum of the rounded squares (see the header) */
            auto tile_sse = [&](uint8_t sbx) {
              float sq[256];
              for (int i = 0; i < 16; ++i)
                for (int t = 0; t < 16; ++t) {
                  int64_t r = r0 + i, k = 16 * kb + t;
                  float y = Y[static_cast<size_t>(r * K + k)];
                  float diff = y - decode_element(encode_element(c, y, sbx, r, k), sbx, ts);
                  sq[i * 16 + t] = diff * diff;
                }
              return quad_sum(sq, 0, 0, 16);
            };
            const float acc6 = tile_sse(sb);
            const uint8_t sb4 = block_scale_byte(ab, 4.0f, ts);
            const float acc4 = tile_sse(sb4);
            sse_plain[static_cast<size_t>(r0)] += acc6;
            if (acc4 < acc6) {
              sb = sb4;
              sse_chosen[static_cast<size_t>(r0)] += acc4;
            } else {
              sse_chosen[static_cast<size_t>(r0)] += acc6;
            }
          }
          scales[(r0 / 16) * KB + kb] = sb;
          for (int64_t r = r0; r < r0 + 16; ++r)
            for (int64_t t = 0; t < 16; ++t) {
              int64_t k = 16 * kb + t;
              store_code(r, k, encode_element(c, Y[static_cast<size_t>(r * K + k)], sb, r, k));
            }
        }
      }
    });
  } else {
    parallel_ranges(R, 1, nthreads, [&](int64_t lo, int64_t hi) {
      for (int64_t r = lo; r < hi; ++r) {
        for (int64_t kb = 0; kb < KB; ++kb) {
          const float *y = &Y[static_cast<size_t>(r * K + 16 * kb)];
          float ab = 0.0f;
          for (int t = 0; t < 16; ++t) ab = std::max(ab, std::fabs(y[t]));
          uint8_t codes[16];
          uint8_t sb = block_scale_byte(ab, 6.0f, ts);
          for (int t = 0; t < 16; ++t) codes[t] = encode_element(c, y[t], sb, r, 16 * kb + t);
          if (fos || search) {
            /* Four-over-Six (targets 6, 4) or the scale search (6, 5.5, 5, 4.5, 4): each target
             * gives a block scale and codes; keep the one with the lowest block SSE (fp32, fused
             * multiply-add in block order); a later target must be strictly lower.  ts is
             * unchanged. */
            static const float kFos[] = {6.0f, 4.0f};
            static const float kSearch[] = {6.0f, 5.5f, 5.0f, 4.5f, 4.0f};
            const float *targets = search ? kSearch : kFos;
            const int nt = search ? 5 : 2;
            float best = 0.0f;
            for (int ti = 0; ti < nt; ++ti) {
              const uint8_t sbx = ti == 0 ? sb : block_scale_byte(ab, targets[ti], ts);
              uint8_t cx[16];
              float acc = 0.0f;
              for (int t = 0; t < 16; ++t) {
                cx[t] = ti == 0 ? codes[t] : encode_element(c, y[t], sbx, r, 16 * kb + t);
                float diff = y[t] - decode_element(cx[t], sbx, ts);
                acc = std::fmaf(diff, diff, acc);
              }
              if (ti == 0) {
                best = acc;
                sse_plain[static_cast<size_t>(r)] += acc;
              } else if (acc < best) {
                best = acc;
                sb = sbx;
                std::memcpy(codes, cx, 16);
              }
            }
            sse_chosen[static_cast<size_t>(r)] += best;
          }
          scales[r * KB + kb] = sb;
          for (int t = 0; t < 16; ++t) store_code(r, 16 * kb + t, codes[t]);
        }
      }
    });
  }
  if (sse2) {
    double a = 0.0, b = 0.0;
    for (int64_t r = 0; r < R; ++r) {
      a += sse_chosen[static_cast<size_t>(r)];
      b += sse_plain[static_cast<size_t>(r)];
    }
    sse2[0] = a;
    sse2[1] = b;
  }
  return 0;
}

float or_tile_sse_2d(const float *tile, int64_t ld, float ts, float T, uint8_t *sb_out) {
  float ab = 0.0f;
  for (int i = 0; i < 16; ++i)
    for (int t = 0; t < 16; ++t) ab = std::max(ab, std::fabs(tile[i * ld + t]));
  const uint8_t sb = block_scale_byte(ab, T, ts);
  QuantCtx c{16, 16, 0u, 0u, 0u, ts};
  float sq[256];
  for (int i = 0; i < 16; ++i)
    for (int t = 0; t < 16; ++t) {
      float y = tile[i * ld + t];
      float diff = y - decode_element(encode_element(c, y, sb, i, t), sb, ts);
      sq[i * 16 + t] = diff * diff;
    }
  if (sb_out) *sb_out = sb;
  return quad_sum(sq, 0, 0, 16);
}

int or_quantize_given_ts(const float *y, int64_t rows, int64_t cols, int64_t ldy, float ts, uint8_t *data,
                         uint8_t *scales, int nthreads) {
  if (cols % 16 != 0 || rows < 0 || ldy < cols) return 2;
  const int64_t KB = cols / 16;
  QuantCtx c{rows, cols, 0u, 0u, 0u, ts};
  parallel_ranges(rows, 1, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t r = lo; r < hi; ++r) {
      for (int64_t kb = 0; kb < KB; ++kb) {
        const float *blk = y + r * ldy + 16 * kb;
        float ab = 0.0f;
        for (int t = 0; t < 16; ++t) ab = std::max(ab, std::fabs(blk[t]));
        const uint8_t sb = block_scale_byte(ab, 6.0f, ts);
        scales[r * KB + kb] = sb;
        for (int t = 0; t < 16; t += 2) {
          const uint8_t lo_code = encode_element(c, blk[t], sb, r, 16 * kb + t);
          const uint8_t hi_code = encode_element(c, blk[t + 1], sb, r, 16 * kb + t + 1);
          data[r * (cols / 2) + 8 * kb + t / 2] = static_cast<uint8_t>(lo_code | (hi_code << 4));
        }
      }
    }
  });
  return 0;
}

int or_dequantize(const uint8_t *data, const uint8_t *scales, float ts, int64_t R, int64_t K,
                  uint32_t flags, float *y) {
  if (K % 16 != 0) return 2;
  const bool block2d = (flags & OR_BLOCK2D) != 0;
  if (block2d && R % 16 != 0) return 2;
  const int64_t KB = K / 16;
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t k = 0; k < K; ++k) {
      uint8_t byte = data[r * (K / 2) + k / 2];
      uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
      uint8_t sb = block2d ? scales[(r / 16) * KB + k / 16] : scales[r * KB + k / 16];
      y[r * K + k] = decode_element(code, sb, ts);
    }
  }
  return 0;
}

int or_gemm_ref(const uint8_t *a_data, const uint8_t *a_scales, float a_ts, uint32_t a_flags,
                const uint8_t *b_data, const uint8_t *b_scales, float b_ts, uint32_t b_flags,
                int64_t M, int64_t N, int64_t K, const int64_t *tiles, int64_t n_tiles,
                double *c, double *bound, int nthreads) {
  if (K % 16 != 0) return 2;
  const int64_t KB = K / 16;
  /* exact element value q * S (binary64 holds it exactly), tensor scale applied at the end */
  auto elem = [&](const uint8_t *d, const uint8_t *s, uint32_t fl, int64_t row, int64_t k) {
    uint8_t byte = d[row * (K / 2) + k / 2];
    uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
    uint8_t sb = (fl & OR_BLOCK2D) ? s[(row / 16) * KB + k / 16] : s[row * KB + k / 16];
    return static_cast<double>(or_e2m1_value(code)) * static_cast<double>(or_e4m3_value(sb));
  };
  const double tsab = static_cast<double>(a_ts) * static_cast<double>(b_ts);
  for (int64_t t = 0; t < n_tiles; ++t) {
    int64_t r0 = tiles[4 * t], c0 = tiles[4 * t + 1], h = tiles[4 * t + 2], w = tiles[4 * t + 3];
    if (r0 < 0 || c0 < 0 || h < 0 || w < 0 || r0 + h > M || c0 + w > N) return 2;
  }
  parallel_ranges(n_tiles, 1, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      int64_t r0 = tiles[4 * t], c0 = tiles[4 * t + 1], h = tiles[4 * t + 2], w = tiles[4 * t + 3];
      std::vector<double> Ad(static_cast<size_t>(h * K)), Bd(static_cast<size_t>(w * K));
      for (int64_t i = 0; i < h; ++i)
        for (int64_t k = 0; k < K; ++k) Ad[static_cast<size_t>(i * K + k)] = elem(a_data, a_scales, a_flags, r0 + i, k);
      for (int64_t j = 0; j < w; ++j)
        for (int64_t k = 0; k < K; ++k) Bd[static_cast<size_t>(j * K + k)] = elem(b_data, b_scales, b_flags, c0 + j, k);
      for (int64_t i = 0; i < h; ++i) {
        for (int64_t j = 0; j < w; ++j) {
          double acc = 0.0, bnd = 0.0;
          const double *ar = &Ad[static_cast<size_t>(i * K)];
          const double *br = &Bd[static_cast<size_t>(j * K)];
          for (int64_t k = 0; k < K; ++k) {
            acc += ar[k] * br[k];
            bnd += std::fabs(ar[k]) * std::fabs(br[k]);
          }
          c[(r0 + i) * N + (c0 + j)] = acc * tsab;
          bound[(r0 + i) * N + (c0 + j)] = bnd * std::fabs(tsab);
        }
      }
    }
  });
  return 0;
}

int or_gemm_w4a16_ref(const uint16_t *a_bf16, int64_t lda, const uint8_t *b_data, const uint8_t *b_scales,
                      float b_ts, uint32_t b_flags, int64_t M, int64_t N, int64_t K, const int64_t *tiles,
                      int64_t n_tiles, double *c, double *bound, int nthreads) {
  /* C = A * B_hat^T with A bf16 (widened exactly) and B_hat the exact NVFP4 decode: every product
   * a * (q * S) is exact in binary64, the K sum rounds at 2^-53, ts_b is applied at the end. */
  if (K % 16 != 0 || lda < K) return 2;
  const int64_t KB = K / 16;
  for (int64_t t = 0; t < n_tiles; ++t) {
    int64_t r0 = tiles[4 * t], c0 = tiles[4 * t + 1], h = tiles[4 * t + 2], w = tiles[4 * t + 3];
    if (r0 < 0 || c0 < 0 || h < 0 || w < 0 || r0 + h > M || c0 + w > N) return 2;
  }
  const double tsb = static_cast<double>(b_ts);
  parallel_ranges(n_tiles, 1, nthreads, [&](int64_t lo, int64_t hi) {
    for (int64_t t = lo; t < hi; ++t) {
      int64_t r0 = tiles[4 * t], c0 = tiles[4 * t + 1], h = tiles[4 * t + 2], w = tiles[4 * t + 3];
      std::vector<double> Ad(static_cast<size_t>(h * K)), Bd(static_cast<size_t>(w * K));
      for (int64_t i = 0; i < h; ++i)
        for (int64_t k = 0; k < K; ++k)
          Ad[static_cast<size_t>(i * K + k)] = static_cast<double>(widen_bf16(a_bf16[(r0 + i) * lda + k]));
      for (int64_t j = 0; j < w; ++j)
        for (int64_t k = 0; k < K; ++k) {
          const int64_t row = c0 + j;
          uint8_t byte = b_data[row * (K / 2) + k / 2];
          uint8_t code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
          uint8_t sb = (b_flags & OR_BLOCK2D) ? b_scales[(row / 16) * KB + k / 16] : b_scales[row * KB + k / 16];
          Bd[static_cast<size_t>(j * K + k)] =
              static_cast<double>(or_e2m1_value(code)) * static_cast<double>(or_e4m3_value(sb));
        }
      for (int64_t i = 0; i < h; ++i) {
        for (int64_t j = 0; j < w; ++j) {
          double acc = 0.0, bnd = 0.0;
          const double *ar = &Ad[static_cast<size_t>(i * K)];
          const double *br = &Bd[static_cast<size_t>(j * K)];
          for (int64_t k = 0; k < K; ++k) {
            acc += ar[k] * br[k];
            bnd += std::fabs(ar[k]) * std::fabs(br[k]);
          }
          c[(r0 + i) * N + (c0 + j)] = acc * tsb;
          bound[(r0 + i) * N + (c0 + j)] = bnd * std::fabs(tsb);
        }
      }
    }
  });
  return 0;
}

} /* extern "C" */
