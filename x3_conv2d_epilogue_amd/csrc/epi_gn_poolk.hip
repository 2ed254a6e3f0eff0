// epi_gn_poolk.hip -- conv3x3 + bias with the GroupNorm-partials epilogue
// and max-pooling windows of size 1..16 other than 4 (4 has its own kernels
// in epi_gn_pool.hip), NCHW x.  Tiles of 16 x 64 outputs trimmed to whole
// windows (dispatch.hpp: gnk_rows, gnk_cols), 8 wavefronts; with Cin <= 16
// and Cout <= 64 the weights of both K chunks stay resident in LDS.
// Windows of 1 and 2 fold inside a wavefront (partials per group of 4
// channels or per channel); windows of 3..16 are combined in LDS
// (per-channel partials).
#include "dispatch.hpp"

namespace x3i {
namespace {

template <int EPI>
x3_status dispatch_poolk(const x3::ConvArgs& a, hipStream_t st) {
  if (rows_aligned16(a)) {
    if (a.Cin <= 16 && a.Cout <= 64)
      return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 2>, EPI>(a, st);
    return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 0>, EPI>(a, st);
  }
  return run_conv<x3::Geo<2, 8, 16, 2, 8, false, 0>, EPI>(a, st);
}

}  // namespace

x3_status launch_gn_poolk(const x3::ConvArgs& a, hipStream_t st) {
  if (a.pk >= 3) return dispatch_poolk<x3::EPI_GN_POOLKL>(a, st);
  return gn_partials_per_channel(a.Cout, a.groups)
             ? dispatch_poolk<x3::EPI_GN_POOLK_CH>(a, st)
             : dispatch_poolk<x3::EPI_GN_POOLK>(a, st);
}

}  // namespace x3i
