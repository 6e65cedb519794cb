// Instantiations of the ring kernel for a transposed A (A stored K x M),
// bf16 and fp16 inputs, both B layouts.
#include "gemm_mfma.h"
#include "gemm_ring.h"

namespace tmm {

namespace {
template <int AB, int CT>
hipError_t ring_ta_layout(bool trans_b, const GemmParams &p, hipStream_t stream) {
  using namespace gemm_detail;
  return trans_b ? launch_ring_ta<AB, CT, true>(p, stream) : launch_ring_ta<AB, CT, false>(p, stream);
}
}  // namespace

hipError_t launch_gemm_ring_ta(Fmt ab, Fmt c, bool trans_b, const GemmParams &p, hipStream_t stream) {
  if (ab == kBF16) return c == kF32 ? ring_ta_layout<kBF16, kF32>(trans_b, p, stream)
                                    : ring_ta_layout<kBF16, kBF16>(trans_b, p, stream);
  if (ab == kF16) return c == kF32 ? ring_ta_layout<kF16, kF32>(trans_b, p, stream)
                                   : ring_ta_layout<kF16, kF16>(trans_b, p, stream);
  return hipErrorInvalidValue;
}

}  // namespace tmm
