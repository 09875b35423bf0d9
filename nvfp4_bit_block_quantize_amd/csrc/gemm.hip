// gemm.hip -- host dispatch of the block-scaled NVFP4 x NVFP4 GEMM (kernels in gemm_kernels.hpp):
// the (group, tile) schedule of a plain or grouped call, the choice of kernel, and the launch of the
// variant instantiated for the output type and the operands' scale layouts.
#include "gemm_kernels.hpp"

namespace nvfp4 {

namespace gemm {
#define NVFP4_DECLARE(OUT, A2D, B2D) \
  extern template hipError_t launch_variant<OUT, A2D, B2D>(const GemmKArgs &, int32_t, bool, bool, bool, hipStream_t);
NVFP4_GEMM_VARIANTS(NVFP4_DECLARE)
#undef NVFP4_DECLARE
}  // namespace gemm

namespace {

using namespace gemm;

hipError_t launch_gemm_variant(int out, bool a2d, bool b2d, const GemmKArgs &p, int32_t grid, bool full, bool paired,
                               bool half, hipStream_t stream) {
#define NVFP4_CASE(OUT, A2D, B2D) \
  if (out == OUT && a2d == A2D && b2d == B2D) return launch_variant<OUT, A2D, B2D>(p, grid, full, paired, half, stream);
  NVFP4_GEMM_VARIANTS(NVFP4_CASE)
#undef NVFP4_CASE
  return hipErrorInvalidValue;
}

// Compute units of the current device (cached per device; 0 if unknown).
int32_t compute_units() {
  static int32_t cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_gemm(const GemmArgs &a) {
  const int32_t G = a.num_groups < 1 ? 1 : a.num_groups;
  const int64_t KB = a.K / 16;
  const int32_t tiles_n = static_cast<int32_t>((a.N + BN - 1) / BN);
  const bool bf16 = a.c_dtype == 1, quant = a.c_dtype == 2;
  const int out = quant ? 2 : (bf16 ? 1 : 0);
  // whole K steps and 8-byte aligned scale rows: branch-free loads (K == 0 takes the generic
  // kernel, whose loads are guarded: the ring's prologue would read the clamped step -1); whole
  // pairs of steps and 16-byte aligned scale rows (K % 256 == 0 makes every row a multiple of 16
  // bytes): scales two steps per load
  const bool full = a.K > 0 && (a.K % 128) == 0 && (reinterpret_cast<uintptr_t>(a.a_scales) & 7u) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.b_scales) & 7u) == 0;
  const bool paired = full && (a.K % 256) == 0 && (reinterpret_cast<uintptr_t>(a.a_scales) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.b_scales) & 15u) == 0;
  // (the entry point admits the quantized output only where the paired pipelined kernel applies)
  if (quant && !paired) return hipErrorInvalidValue;
  // Grouped calls with the paired kernel and fp32 or bf16 C: a group whose last 256-row band holds
  // at most 128 rows gets that band as 128 x 256 tiles of half the cost, in a second launch after
  // the full tiles, so that the groups' ragged ends neither double their work nor add a round of
  // full tiles.
  const bool halves = a.num_groups > 1 && paired && out != 2;
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
    p.q_data = a.q_data;
    p.q_scales = a.q_scales;
    p.q_ts = a.q_ts;
    p.amax = a.amax;
    p.vec_store = (reinterpret_cast<uintptr_t>(a.c) % 16) == 0 && ((a.ldc * (bf16 ? 2 : 4)) % 16) == 0;
    GemmKArgs ph = p;  // the half tiles' launch
    int32_t tiles = 0, half_tiles = 0;
    for (int32_t g = 0; g < ng; ++g) {
      const int64_t r0 = a.group_offsets ? a.group_offsets[g0 + g] : 0;
      const int64_t r1 = a.group_offsets ? a.group_offsets[g0 + g + 1] : a.M;
      int64_t bands = ((r1 - r0) + BM - 1) / BM;
      const bool half = halves && bands > 0 && (r1 - r0) - (bands - 1) * BM <= BM / 2;
      if (half) --bands;
      p.row_begin[g] = r0;
      p.row_end[g] = r1;
      p.tile_begin[g] = tiles;
      tiles += static_cast<int32_t>(bands) * tiles_n;
      ph.row_begin[g] = r0 + bands * BM;
      ph.row_end[g] = r1;
      ph.tile_begin[g] = half_tiles;
      half_tiles += half ? tiles_n : 0;
    }
    p.row_begin[ng] = a.group_offsets ? a.group_offsets[g0 + ng] : a.M;
    p.tile_begin[ng] = tiles;
    p.total_tiles = tiles;
    ph.row_begin[ng] = p.row_begin[ng];
    ph.tile_begin[ng] = half_tiles;
    ph.total_tiles = half_tiles;
    // The pipelined kernel with bf16 C (or fp32 C, paired) and at least four K steps runs each workgroup over several
    // tiles (one workgroup per compute unit, a multiple of 8 so that every workgroup keeps its XCD):
    // the next tile's first steps load under the last steps of the current one, and no workgroup
    // launch separates them.  Otherwise one workgroup per tile.
    auto grid_for = [&](int32_t n) {
      int32_t grid = n;
      if (full && (out == 1 || (out == 0 && paired)) && a.K / 128 >= 4) {
        const int32_t cus = compute_units() / 8 * 8;
        if (cus >= 8 && cus < n) grid = cus;
      }
      return grid;
    };
    // (K == 0 still launches: the K loop is empty and C = 0)
    if (tiles > 0) {
      hipError_t err = launch_gemm_variant(out, a.a_2d, a.b_2d, p, grid_for(tiles), full, paired, false, a.stream);
      if (err != hipSuccess) return err;
    }
    if (half_tiles > 0) {
      hipError_t err = launch_gemm_variant(out, a.a_2d, a.b_2d, ph, grid_for(half_tiles), full, paired, true, a.stream);
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

}  // namespace nvfp4
