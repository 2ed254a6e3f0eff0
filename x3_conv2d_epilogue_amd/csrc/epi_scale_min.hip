// epi_scale_min.hip -- conv3x3 + bias, scalar scale, channel minimum.
#include "dispatch.hpp"

namespace x3i {
x3_status launch_scale_min(const x3::ConvArgs& a, hipStream_t st) {
  return dispatch<x3::EPI_SCALE_MIN>(a, st);
}
}  // namespace x3i
