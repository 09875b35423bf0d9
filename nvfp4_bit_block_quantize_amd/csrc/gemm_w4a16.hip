// gemm_w4a16.hip -- bf16 activations x NVFP4 weights on the gfx950 matrix cores (the weight-only
// 4-bit path that serving stacks fall back to on hardware without a native FP4 x FP4 product; NVIDIA
// Hopper in the pages' account of the Nemotron 3 Ultra NVFP4 checkpoint).
//
// C[i][j] = ts_b * sum_k a_ik (q_jk S_jk).  Each weight element is decoded exactly to bf16 with its
// block scale folded in: q (E2M1, <= 2 significant bits) times S (E4M3, <= 4 bits) has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in bf16 (8 bits, normal from 2^-126).
// v_mfma_f32_32x32x16_bf16 then forms exact products of bf16 pairs and accumulates them in fp32;
// ts_b is applied once in the epilogue.
//
// Decode of 8 codes (one dword): v_cvt_scalef32_pk_f32_fp4 (scale 1.0) gives two exact fp32 values
// per instruction, v_mul_f32 by S, v_cvt_pk_bf16_f32 packs two (exact): two VALU ops per element.
//
// Tiling follows the NVFP4 x NVFP4 kernel: a 256-thread workgroup owns a 256 x 256 tile of C, its
// four waves a 128 x 128 quarter each (4 x 4 MFMA tiles of 32 x 32).  K advances 64 per step through
// a ring of three LDS stages filled by direct global->LDS loads two steps ahead:
//   A       [256 rows][128 B] bf16, 16-byte chunk c of row r at position c ^ ((r + ((r >> 3) & 3)) & 7)
//   B codes [256 rows][32 B],       16-byte chunk c of row r at position c ^ (((r >> 2) ^ (r >> 3)) & 1)
//   B scales [256 rows][4 B]        (the four E4M3 block scales of the step)
// (the swizzles make the fragment reads conflict-free ds_read_b128s).  Within a step, lane half h
// and sub-step s = 0..3 take K [32 h + 8 s, 32 h + 8 s + 8) for both operands: an A chunk, a dword
// of the B chunk, and B block scale 2 h + s / 2.
#include "gemm_common.hpp"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace gemm;

constexpr int kWA = 0, kWB = 32768, kWS = 40960, kWStage = 41984;  // stage layout (bytes)
// direct loads per lane and step: 8 for A, 2 for B codes, 1 for B scales; 6 of them are issued in
// sub-steps 0 and 1, before the step's barrier
constexpr int kWLoadsBeforeBarrier = 6;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct W4Args {
  const uint8_t *a;
  int64_t lda_bytes;
  int64_t M;
  const uint8_t *b_data, *b_scales;
  const float *b_ts;
  int64_t N, K;
  uint8_t *c;
  int64_t ldc;
  int32_t tiles_n, total_tiles;
  int32_t vec_store;
};

// Both swizzles depend on the low 5 bits of the row only, so that the 32-row fragments of a wave all
// see the same pattern.
__device__ __forceinline__ uint32_t swz_a(uint32_t r) { return (r + ((r >> 3) & 3u)) & 7u; }
__device__ __forceinline__ uint32_t swz_b(uint32_t r) { return ((r >> 2) ^ (r >> 3)) & 1u; }

// 8 codes (code n at bits 4n) times the fp32 block scale S -> 8 exact bf16 values.
__device__ __forceinline__ bf16x8 decode8_bf16(uint32_t w, float S) {
  const float2v q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float2v q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const float2v q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const float2v q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  const bf16x2v v0 = __builtin_convertvector((float2v){q0[0] * S, q0[1] * S}, bf16x2v);
  const bf16x2v v1 = __builtin_convertvector((float2v){q1[0] * S, q1[1] * S}, bf16x2v);
  const bf16x2v v2 = __builtin_convertvector((float2v){q2[0] * S, q2[1] * S}, bf16x2v);
  const bf16x2v v3 = __builtin_convertvector((float2v){q3[0] * S, q3[1] * S}, bf16x2v);
  const u32x4 bits = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                      __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
  return __builtin_bit_cast(bf16x8, bits);
}

template <bool OUT_BF16, bool B2D>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4a16_kernel(W4Args p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * kWStage];

  const int32_t tile = xcd_tile(blockIdx.x, p.total_tiles);
  int32_t tm, tn;
  band_tile(tile, p.tiles_n, p.total_tiles / p.tiles_n, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * BN;
  const int64_t KT = p.K / 64, KB = p.K / 16, row_bytes = p.K / 2;

  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t h = lane >> 5, l32 = lane & 31u;
  const uint32_t wm = (wave >> 1) * 128, wn = (wave & 1) * 128;

  floatx16 acc[4][4];  // [B fragment j][A fragment i]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

  if (KT > 0) {
    // ---- direct-load sources (32-bit offsets from per-step bases; each operand is below 4 GiB).
    // Wave w fetches tile rows [64 w, 64 w + 64) of A (8 rows per load), of the B codes (32 rows
    // per load) and of the B scales (one dword per row).  Rows beyond the operand read some valid
    // row: their products reach only outputs that are never stored.
    uint32_t srcA[8], srcB[2], srcS;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t R = 64 * wave + 8 * i + (lane >> 3);
      const uint32_t c = (lane & 7u) ^ swz_a(R);  // logical chunk stored at position lane & 7
      // rows beyond M read a valid row chosen modulo M (not all the last row: many lanes on one
      // address are slow)
      const int64_t ra = m0 + R < p.M ? m0 + R : (m0 + R) % p.M;
      srcA[i] = static_cast<uint32_t>(ra * p.lda_bytes + 16 * c);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t R = 64 * wave + 32 * i + (lane >> 1);
      const uint32_t c = (lane & 1u) ^ swz_b(R);
      srcB[i] = static_cast<uint32_t>(min(n0 + R, p.N - 1) * row_bytes + 16 * c);
    }
    {
      const int64_t r = min(n0 + 64 * wave + lane, p.N - 1);
      srcS = static_cast<uint32_t>(B2D ? (r / 16) * KB : r * KB);
    }
    // load q (0..10) of step kt into stage st; steps beyond K re-fetch the last step into a stage
    // that is never consumed
    auto load = [&](uint8_t *st, int64_t kt, int q) {
      const int64_t kc = kt < KT ? kt : KT - 1;
      if (q < 8)
        lds_load16(p.a + kc * 128 + srcA[q], st + kWA + (64 * wave + 8 * q) * 128);
      else if (q < 10)
        lds_load16(p.b_data + kc * 32 + srcB[q - 8], st + kWB + (64 * wave + 32 * (q - 8)) * 32);
      else
        lds_load4(p.b_scales + kc * 4 + srcS, st + kWS + 64 * wave * 4);
    };

    // ---- fragment reads (a wave's fragment rows share their low 5 bits with l32, so the swizzles
    // depend on the lane only)
    const uint32_t rdA = kWA + (wm + l32) * 128, rdB = kWB + (wn + l32) * 32, rdS = kWS + (wn + l32) * 4;
    const uint32_t swa = swz_a(l32), posB = 16 * (h ^ swz_b(l32));
    auto read_a = [&](const uint8_t *st, int s, bf16x8 (&af)[4]) {
      const uint32_t pos = 16 * ((4 * h + s) ^ swa);
#pragma unroll
      for (int f = 0; f < 4; ++f) af[f] = *reinterpret_cast<const bf16x8 *>(st + rdA + 4096 * f + pos);
    };
    // B codes of the step (this lane's 32) and the scale dword of each fragment row
    auto read_b = [&](const uint8_t *st, uint4 (&cb)[4], uint32_t (&sw)[4]) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        cb[f] = *reinterpret_cast<const uint4 *>(st + rdB + 1024 * f + posB);
        sw[f] = *reinterpret_cast<const uint32_t *>(st + rdS + 128 * f);
      }
    };
    // fp32 scales of this lane's two blocks 2 h, 2 h + 1 of the step
    auto scales = [&](const uint32_t (&sw)[4], float (&s_lo)[4], float (&s_hi)[4]) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const float2v v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[f] >> (16 * h), 1.0f, false);
        s_lo[f] = v[0];
        s_hi[f] = v[1];
      }
    };

    uint8_t *const st0 = smem, *const st1 = smem + kWStage;
#pragma unroll
    for (int q = 0; q < 11; ++q) load(st0, 0, q);
#pragma unroll
    for (int q = 0; q < 11; ++q) load(st1, 1, q);
    wait_vmcnt<11>();
    lds_barrier();
    uint4 cb[4], cbn[4];  // B codes of this step / the next
    uint32_t swn[4];      // the next step's raw scale dwords
    float s_lo[4], s_hi[4];
    bf16x8 afc[4], bfc[4], a3[4], an0[4];
    read_b(st0, cb, swn);
    read_a(st0, 0, afc);
    scales(swn, s_lo, s_hi);
#pragma unroll
    for (int f = 0; f < 4; ++f) bfc[f] = decode8_bf16(cb[f].x, s_lo[f]);

    // One K step out of stage cur: four sub-steps of 16 MFMAs, each decoding the B fragments of the
    // next sub-step under its MFMAs.  The loads of step kt + 2 into tgt are spread over the
    // sub-steps (3, 3, 3, 2).  The step's barrier follows sub-step 1, once the A fragments of
    // sub-steps 2 and 3 are in registers; the next step's codes, scales and first A fragments are
    // read right after it, two sub-steps before their first use.
    auto step = [&](uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt, uint8_t *__restrict__ tgt, int64_t kt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int q = 3 * s; q < (s < 3 ? 3 * s + 3 : 11); ++q) load(tgt, kt + 2, q);
        bf16x8 afn[4], bfn[4];
        if (s == 0) {
          read_a(cur, 1, afn);
        } else if (s == 1) {
          read_a(cur, 2, afn);
          read_a(cur, 3, a3);
        }
        if (s == 3) scales(swn, s_lo, s_hi);  // the next step's (this step's are dead)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (s == 2) afn[f] = a3[f];
          if (s == 3) afn[f] = an0[f];
          bfn[f] = s < 3 ? decode8_bf16(pick(cb[f], s + 1), s + 1 < 2 ? s_lo[f] : s_hi[f])
                         : decode8_bf16(cbn[f].x, s_lo[f]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfc[j], afc[i], acc[j][i], 0, 0, 0);
        // one MFMA, then up to five VALU instructions (the 64 of the decode and the address and scale
        // arithmetic): the matrix pipe is never left behind a long run of VALU work (a wave issues
        // in order)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          afc[f] = afn[f];
          bfc[f] = bfn[f];
        }
        if (s == 1) {
          // every read of this stage is issued, and this lane's loads of step kt + 1 have landed:
          // after the barrier the next stage is complete and this one may be refilled
          wait_vmcnt<kWLoadsBeforeBarrier>();
          wait_lgkmcnt0();
          lds_barrier();
          read_b(nxt, cbn, swn);
          read_a(nxt, 0, an0);
        }
        if (s == 3) {
#pragma unroll
          for (int f = 0; f < 4; ++f) cb[f] = cbn[f];
        }
      }
    };
    uint8_t *cur = st0, *nxt = st1, *tgt = smem + 2 * kWStage;
    for (int64_t kt = 0; kt < KT; ++kt) {
      step(cur, nxt, tgt, kt);
      uint8_t *const done = cur;
      cur = nxt;
      nxt = tgt;
      tgt = done;
    }
  }

  store_c_tile<OUT_BF16>(acc, smem, p.c, p.ldc, m0, n0, p.M, p.N, *p.b_ts, 1.0f, p.vec_store != 0, wave, lane);
}

// ---- few activation rows (decode): weight streaming --------------------------------------------------
// With M <= 64 the product is bound by reading the weight once from HBM.  A workgroup of W waves owns
// 64 weight rows (four 16-row tiles) and 16 MT activation rows (all of them for M <= 64; for M up
// to 256 the grid's second dimension walks 64-row chunks, each a pass over the weight, the later
// ones mostly from the Infinity Cache); its waves split K, wave w
// taking the 128-element chunks w, w + W, ... (neighbouring waves read neighbouring bytes of each row),
// and their partial sums meet in LDS at the end.
// Per chunk and lane (n = l & 15, g = l >> 4):
//   - the weight tile's codes arrive as one 16-byte load per lane (row n, codes [32 g, 32 g + 32)),
//     i.e. dword j holds K offsets 32 g + 8 j; a 4 x 4 transpose across the four 16-lane rows
//     (v_permlane32_swap, then v_permlane16_swap) gives dword t = K offsets 32 t + 8 g;
//   - the activation chunk (16 MT rows x 256 bytes) arrives lane-contiguously (load t of M tile mt: rows
//     16 mt + 4 t + (l >> 4), 16-byte piece l & 15), passes through a wave-private LDS buffer (piece j
//     of row r at position j ^ (r & 15): conflict-free both ways) and is read back as MFMA fragments:
//     row m = l & 15, piece 4 t + g = K offsets 32 t + 8 g;
//   - MFMA t (v_mfma_f32_16x16x32_bf16) consumes K offsets {32 t + 8 g + e}: the same set on both sides.
// The block scale of (t, g) is block 2 t + (g >> 1) of the chunk's eight.
constexpr int kSkRows = 64;
// buffer resource word 3 for gfx9-family raw buffer loads (32-bit data format), and a byte offset
// beyond any buffer used here (each is below 2 GiB)
constexpr int32_t kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kSkRed = 4 * 64 + 16;  // floats per (wave, M tile, weight tile) partial (padded)

struct SkArgs {
  const uint8_t *a;
  int64_t lda_bytes;
  int64_t M;
  const uint8_t *b_data, *b_scales;
  const float *b_ts;
  int64_t N, K;
  uint8_t *c;
  int64_t ldc;
};

template <int MT>
struct SkChunk {
  uint4 b[4];       // codes of the four weight tiles (before the transpose)
  uint2 s[4];       // the chunk's eight scale bytes per tile row
  uint4 a[MT][4];   // activation rows, lane-contiguous
};

typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int MT, int W, int R, bool OUT_BF16, bool B2D>
__global__ __launch_bounds__(64 * W, 1) void gemm_w4a16_skinny_kernel(SkArgs p) {
  __shared__ float red[W * MT * 4 * kSkRed];
  __shared__ __attribute__((aligned(16))) uint8_t a_tr[W][16 * MT * 256];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t n16 = lane & 15u, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kSkRows;
  const uint32_t m_base = 16 * MT * blockIdx.y;  // this workgroup's activation rows
  const int64_t KC = p.K / 128, KB = p.K / 16, row_bytes = p.K / 2;

  // per-lane sources: 32-bit byte offsets of chunk 0 (each operand is below 4 GiB)
  uint32_t srcB[4], srcS[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t n = min(n0 + 16 * nt + n16, p.N - 1);
    srcB[nt] = static_cast<uint32_t>(n * row_bytes + 16 * g);
    srcS[nt] = static_cast<uint32_t>(B2D ? (n / 16) * KB : n * KB);
  }
  // activation rows m_base + 16 mt + 4 t + (l >> 4); rows beyond M read a valid row chosen modulo M
  // (their sums are never stored)
  const uint32_t a_rows = static_cast<uint32_t>(p.M), a_r0 = lane >> 4, a_piece = 16 * (lane & 15);
  const uint32_t lda_b = static_cast<uint32_t>(p.lda_bytes);
  uint32_t a_off[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t r = m_base + 16 * mt + 4 * t + a_r0;
      a_off[mt][t] = (r < a_rows ? r : r % a_rows) * lda_b + a_piece;
    }
  // v_perm selector picking scale bytes 2 t + (g >> 1), t = 0..3, out of the chunk's eight
  const uint32_t sh = g >> 1;
  const uint32_t ssel = sh | ((2 + sh) << 8) | ((4 + sh) << 16) | ((6 + sh) << 24);

  // Loads are buffer loads: a chunk index past this wave's last turns into an offset beyond the
  // buffer, which the hardware answers with zeros and no memory access.  So every iteration issues
  // the same loads (the wait counts stay exact) and a padding chunk adds zeros.
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.b_data), 0, static_cast<int32_t>(p.N * row_bytes), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.b_scales), 0, static_cast<int32_t>((B2D ? (p.N + 15) / 16 : p.N) * KB), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(p.a), 0, static_cast<int32_t>((p.M - 1) * p.lda_bytes + 2 * p.K), kBufferWord3);
  auto load = [&](SkChunk<MT> &ch, int64_t c, bool valid) {
    const uint32_t ob = valid ? static_cast<uint32_t>(c * 64) : kOutOfRange;
    const uint32_t os = valid ? static_cast<uint32_t>(c * 8) : kOutOfRange;
    const uint32_t oa = valid ? static_cast<uint32_t>(c * 256) : kOutOfRange;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      ch.b[nt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_b, srcB[nt] + ob, 0, 0));
      ch.s[nt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs_s, srcS[nt] + os, 0, 0));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        ch.a[mt][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs_a, a_off[mt][t] + oa, 0, 0));
  };
  // activation chunk -> this wave's LDS buffer -> MFMA fragments (see above)
  uint8_t *const tr = a_tr[wave];
  const uint32_t rd_row = 256 * n16;
  auto fragments = [&](const SkChunk<MT> &ch, uint4 (&af)[MT][4]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // row 16 mt + 4 t + (l >> 4): (row & 15) = 4 t + (l >> 4)
        const uint32_t row = 16 * mt + 4 * t + (lane >> 4);
        *reinterpret_cast<uint4 *>(tr + 256 * row + (16 * ((lane & 15) ^ (4 * t + (lane >> 4))))) = ch.a[mt][t];
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[mt][t] = *reinterpret_cast<const uint4 *>(tr + 4096 * mt + rd_row + 16 * ((4 * t + g) ^ n16));
  };

  floatx4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](const SkChunk<MT> &ch) {
    uint4 af[MT][4];
    fragments(ch, af);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // 4 x 4 transpose of the tile's dwords across the lane rows g
      uint32_t x0 = ch.b[nt].x, x1 = ch.b[nt].y, x2 = ch.b[nt].z, x3 = ch.b[nt].w;
      {
        const auto r02 = __builtin_amdgcn_permlane32_swap(x0, x2, false, false);
        const auto r13 = __builtin_amdgcn_permlane32_swap(x1, x3, false, false);
        const auto r01 = __builtin_amdgcn_permlane16_swap(r02[0], r13[0], false, false);
        const auto r23 = __builtin_amdgcn_permlane16_swap(r02[1], r13[1], false, false);
        x0 = r01[0];
        x1 = r01[1];
        x2 = r23[0];
        x3 = r23[1];
      }
      const uint32_t sb = __builtin_amdgcn_perm(ch.s[nt].y, ch.s[nt].x, ssel);
      const float2v s01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false);
      const float2v s23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, true);
      const bf16x8 w[4] = {decode8_bf16(x0, s01[0]), decode8_bf16(x1, s01[1]), decode8_bf16(x2, s23[0]),
                           decode8_bf16(x3, s23[1])};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[mt][t]), w[t],
                                                                acc[mt][nt], 0, 0, 0);
    }
  };

  // this wave's chunks: wave, wave + W, ...; a ring of R register sets keeps the loads of R - 1 chunks
  // in flight under the math (the scheduling barriers keep each chunk's loads ahead of the math
  // before them).  The count is rounded up to a multiple of R; padding chunks load zeros.
  const int64_t nch = wave < KC ? (KC - wave + W - 1) / W : 0;
  {
    auto chunk = [&](int64_t i) { return static_cast<int64_t>(wave) + W * i; };
    SkChunk<MT> ring[R];
#pragma unroll
    for (int j = 0; j < R - 1; ++j) load(ring[j], chunk(j), j < nch);
    for (int64_t i = 0; i < nch; i += R) {
#pragma unroll
      for (int j = 0; j < R; ++j) {
        load(ring[(j + R - 1) % R], chunk(i + j + R - 1), i + j + R - 1 < nch);
        __builtin_amdgcn_sched_barrier(0);
        compute(ring[j]);
      }
    }
  }

  // partial sums -> LDS; lane l of tile (mt, nt) holds rows 4 g + i, column n16
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * MT + mt) * 4 + nt) * kSkRed + 64 * i + lane] = acc[mt][nt][i];
  __syncthreads();
  // thread (r = tid >> 6, col = tid & 63) sums rows r, r + W, ... of every M tile over the waves
  const float ts = *p.b_ts;
  const uint32_t col = threadIdx.x & 63u, r0 = threadIdx.x >> 6, nt = col >> 4;
  const int64_t n = n0 + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int h = 0; h < 16 / W; ++h) {
      const uint32_t mr = r0 + W * h;  // row within the M tile
      const int64_t m = m_base + 16 * mt + mr;
      const uint32_t off = (mt * 4 + nt) * kSkRed + 64 * (mr & 3) + (col & 15) + 16 * (mr >> 2);
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) v += red[w * MT * 4 * kSkRed + off];
      v *= ts;
      if (m < p.M && n < p.N) {
        if constexpr (OUT_BF16)
          reinterpret_cast<uint16_t *>(p.c + m * p.ldc * 2)[n] = static_cast<uint16_t>(bf16_rne(v));
        else
          reinterpret_cast<float *>(p.c + m * p.ldc * 4)[n] = v;
      }
    }
}

// Four waves (one per SIMD) and two chunks per ring: measured on the 16 x 14336 x 4096 decode shape,
// eight waves or deeper rings were no faster (deeper rings delay every wave's first chunk)
template <int MT>
void launch_skinny(const W4A16Args &a, const SkArgs &p) {
  constexpr int W = 4, R = 2;
  const dim3 grid(static_cast<uint32_t>((a.N + kSkRows - 1) / kSkRows),
                  static_cast<uint32_t>((a.M + 16 * MT - 1) / (16 * MT))),
      block(64 * W);
  if (a.c_dtype == 1) {
    if (a.b_2d) hipLaunchKernelGGL((gemm_w4a16_skinny_kernel<MT, W, R, true, true>), grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL((gemm_w4a16_skinny_kernel<MT, W, R, true, false>), grid, block, 0, a.stream, p);
  } else {
    if (a.b_2d) hipLaunchKernelGGL((gemm_w4a16_skinny_kernel<MT, W, R, false, true>), grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL((gemm_w4a16_skinny_kernel<MT, W, R, false, false>), grid, block, 0, a.stream, p);
  }
}

}  // namespace

hipError_t launch_gemm_w4a16(const W4A16Args &a) {
  // few activation rows, whole 128-element chunks, 8-byte aligned scale rows: weight streaming,
  // one pass over the weight per 64 activation rows (up to 256 rows: beyond, the tiled kernel's
  // single pass over the weight wins)
  if (a.M > 0 && a.M <= 256 && a.N > 0 && a.K > 0 && a.K % 128 == 0 &&
      (reinterpret_cast<uintptr_t>(a.b_scales) & 7u) == 0 && (a.M - 1) * a.lda * 2 + 2 * a.K < (int64_t(1) << 31)) {
    SkArgs p{};
    p.a = static_cast<const uint8_t *>(a.a);
    p.lda_bytes = a.lda * 2;
    p.M = a.M;
    p.b_data = a.b_data;
    p.b_scales = a.b_scales;
    p.b_ts = a.b_ts;
    p.N = a.N;
    p.K = a.K;
    p.c = static_cast<uint8_t *>(a.c);
    p.ldc = a.ldc;
    switch (a.M <= 64 ? (a.M + 15) / 16 : 4) {
      case 1: launch_skinny<1>(a, p); break;
      case 2: launch_skinny<2>(a, p); break;
      case 3: launch_skinny<3>(a, p); break;
      default: launch_skinny<4>(a, p); break;
    }
    return hipGetLastError();
  }
  const int32_t tiles_n = static_cast<int32_t>((a.N + BN - 1) / BN);
  const int32_t tiles_m = static_cast<int32_t>((a.M + BM - 1) / BM);
  if (tiles_n == 0 || tiles_m == 0) return hipSuccess;
  W4Args p{};
  p.a = static_cast<const uint8_t *>(a.a);
  p.lda_bytes = a.lda * 2;
  p.M = a.M;
  p.b_data = a.b_data;
  p.b_scales = a.b_scales;
  p.b_ts = a.b_ts;
  p.N = a.N;
  p.K = a.K;
  p.c = static_cast<uint8_t *>(a.c);
  p.ldc = a.ldc;
  p.tiles_n = tiles_n;
  p.total_tiles = tiles_n * tiles_m;
  const bool bf16 = a.c_dtype == 1;
  p.vec_store = (reinterpret_cast<uintptr_t>(a.c) % 16) == 0 && ((a.ldc * (bf16 ? 2 : 4)) % 16) == 0;
  const dim3 grid(p.total_tiles), block(kThreads);
  if (bf16) {
    if (a.b_2d) hipLaunchKernelGGL((gemm_w4a16_kernel<true, true>), grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL((gemm_w4a16_kernel<true, false>), grid, block, 0, a.stream, p);
  } else {
    if (a.b_2d) hipLaunchKernelGGL((gemm_w4a16_kernel<false, true>), grid, block, 0, a.stream, p);
    else hipLaunchKernelGGL((gemm_w4a16_kernel<false, false>), grid, block, 0, a.stream, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
