// Instantiations of the MFMA GEMM kernel for f8 inputs (one translation
// unit per input type so the kernels build in parallel).
#include "gemm_mfma.h"
#include "gemm_ring.h"
#include "gemm_quad8.h"

namespace tmm {

hipError_t launch_gemm_f8(Fmt c, bool trans_b, Tile tile, bool vec, const GemmParams &p,
                          hipStream_t stream) {
  using namespace gemm_detail;
  return c == kF32 ? launch_layout<kF8, kF32>(trans_b, tile, vec, p, stream)
                   : launch_layout<kF8, kBF16>(trans_b, tile, vec, p, stream);
}

}  // namespace tmm
