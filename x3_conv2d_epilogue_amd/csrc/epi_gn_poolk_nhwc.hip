// epi_gn_poolk_nhwc.hip -- the kernels of epi_gn_poolk.hip for NHWC
// (channels-last) x and pooled output.  Only the 16-byte channel-half
// staging (Cin % 4 == 0, x and w 16-byte aligned): the pixel-major 4-byte
// form of this tile leaves no LDS for the window buffer.
#include "dispatch.hpp"

namespace x3i {
namespace {

template <int EPI>
x3_status dispatch_poolk_nhwc(const x3::ConvArgs& a, hipStream_t st) {
  if (!nhwc_aligned16(a))
    return fail(X3_EUNSUPPORTED,
                "NHWC GroupNorm with pool window %d needs Cin %% 4 == 0 and "
                "16-byte aligned x and weights", a.pk);
  if (a.Cin <= 16 && a.Cout <= 64)
    return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 2, true>, EPI>(a, st);
  return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 0, true>, EPI>(a, st);
}

}  // namespace

x3_status launch_gn_poolk_nhwc(const x3::ConvArgs& a, hipStream_t st) {
  if (a.pk >= 3) return dispatch_poolk_nhwc<x3::EPI_GN_POOLKL>(a, st);
  return gn_partials_per_channel(a.Cout, a.groups)
             ? dispatch_poolk_nhwc<x3::EPI_GN_POOLK_CH>(a, st)
             : dispatch_poolk_nhwc<x3::EPI_GN_POOLK>(a, st);
}

}  // namespace x3i
