// epi_min_tanh2.hip -- conv3x3 + bias, channel minimum, tanh twice.
#include "dispatch.hpp"

namespace x3i {
x3_status launch_min_tanh2(const x3::ConvArgs& a, hipStream_t st) {
  return dispatch<x3::EPI_MIN_TANH2>(a, st);
}
}  // namespace x3i
