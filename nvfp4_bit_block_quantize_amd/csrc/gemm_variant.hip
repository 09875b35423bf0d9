// gemm_variant.hip -- explicit instantiation of one NVFP4 x NVFP4 GEMM variant (output type
// NVFP4_OUT: 0 fp32, 1 bf16, 2 NVFP4; NVFP4_A2D / NVFP4_B2D: 16x16-tile scales of A / B).  The build
// compiles this file once per combination, so the kernel instances compile in parallel.
#include "gemm_kernels.hpp"

#if !defined(NVFP4_OUT) || !defined(NVFP4_A2D) || !defined(NVFP4_B2D)
#error "gemm_variant.hip is compiled with -DNVFP4_OUT=<0|1|2> -DNVFP4_A2D=<0|1> -DNVFP4_B2D=<0|1>"
#endif

namespace nvfp4 {
namespace gemm {
template hipError_t launch_variant<NVFP4_OUT, (NVFP4_A2D != 0), (NVFP4_B2D != 0)>(const GemmKArgs &, int32_t, bool,
                                                                                  bool, bool, hipStream_t);
}  // namespace gemm
}  // namespace nvfp4
