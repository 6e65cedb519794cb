// Instantiations of the MFMA GEMM kernel for f32 inputs (one translation
// unit per input type so the kernels build in parallel).
#include "gemm_mfma.h"

namespace tmm {

hipError_t launch_gemm_f32(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                          hipStream_t stream) {
  using namespace gemm_detail;
  return launch_layout<kF32, kF32>(trans_b, tile, vec, p, stream);
}

}  // namespace tmm
