// epi_mul_lrelu_gelu_tanh.hip -- conv3x3 + bias, per-channel multiplier,
// LeakyReLU, tanh-approximation GELU.
#include "dispatch.hpp"

namespace x3i {
x3_status launch_mul_lrelu_gelu_tanh(const x3::ConvArgs& a, hipStream_t st) {
  return dispatch<x3::EPI_MUL_LRELU_GELU_TANH>(a, st);
}
}  // namespace x3i
