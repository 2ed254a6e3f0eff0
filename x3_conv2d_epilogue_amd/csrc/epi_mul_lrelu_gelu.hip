// epi_mul_lrelu_gelu.hip -- conv3x3 + bias, per-channel multiplier,
// LeakyReLU, exact (erf) GELU.
#include "dispatch.hpp"

namespace x3i {
x3_status launch_mul_lrelu_gelu(const x3::ConvArgs& a, hipStream_t st) {
  return dispatch<x3::EPI_MUL_LRELU_GELU>(a, st);
}
}  // namespace x3i
