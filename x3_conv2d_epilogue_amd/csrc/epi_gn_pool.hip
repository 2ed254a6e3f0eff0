// epi_gn_pool.hip -- conv3x3 + bias with the GroupNorm-partials and
// pooling-window epilogue, and the GroupNorm finalize pass.
#include "dispatch.hpp"

namespace x3i {
namespace {

// GroupNorm path geometry.  With Cin <= 8 and Cout <= 64 (one K chunk, one
// channel block) the weight tile is resident and two 4-wave workgroups
// share a CU; otherwise the 8-wave tiles with 64-channel blocks.  Both have
// 4-row wave tiles (one row of pooling windows).
struct GnGeo {
  int th, twc, nwave;
};
bool gn_resident(int Cin, int Cout) { return Cin <= 8 && Cout <= 64; }
GnGeo gn_geo(int Wo, int Cin, int Cout) {
  if (gn_resident(Cin, Cout)) {
    if (Wo > 64) return {4, 128, 4};
    if (Wo > 32) return {8, 64, 4};
    return {16, 32, 4};
  }
  if (Wo > 128) return {4, 256, 8};
  if (Wo > 64) return {8, 128, 8};
  if (Wo > 32) return {16, 64, 8};
  return {32, 32, 8};
}

template <bool X4, int EPI>
x3_status dispatch_gn(const x3::ConvArgs& a, hipStream_t st) {
  if (gn_resident(a.Cin, a.Cout)) {
    if (a.Wo > 64) return run_conv<x3::Geo<2, 8, 4, 4, 4, X4, 1>, EPI>(a, st);
    if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 8, 2, 4, X4, 1>, EPI>(a, st);
    return run_conv<x3::Geo<2, 8, 16, 1, 4, X4, 1>, EPI>(a, st);
  }
  return dispatch_mt2<EPI, X4>(a, st);
}

}  // namespace

int gn_pps(int Ho, int Wo, int Cin, int Cout) {
  const GnGeo g = gn_geo(Wo, Cin, Cout);
  return ((Ho + g.th - 1) / g.th) * ((Wo + g.twc - 1) / g.twc) * g.nwave;
}

x3_status launch_gn_pool(const x3::ConvArgs& a, hipStream_t st) {
  const bool x4 = rows_aligned16(a);
  if (gn_partials_per_channel(a.Cout, a.groups))
    return x4 ? dispatch_gn<true, x3::EPI_GN_POOL_CH>(a, st)
              : dispatch_gn<false, x3::EPI_GN_POOL_CH>(a, st);
  return x4 ? dispatch_gn<true, x3::EPI_GN_POOL>(a, st)
            : dispatch_gn<false, x3::EPI_GN_POOL>(a, st);
}

x3_status launch_gn_finalize(const x3::GnFinArgs& f, int nblocks,
                             hipStream_t st) {
  // A group of up to 4 channels moves its pooled block as float4 when the
  // block is 16-byte aligned (`out` aligned, block a multiple of 4 floats).
  if (((uintptr_t)f.out & 15u) == 0 && (f.cpg * f.plane) % 4 == 0)
    hipLaunchKernelGGL((x3::gn_finalize_kernel<256, true>), dim3((unsigned)nblocks),
                       dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL((x3::gn_finalize_kernel<256, false>),
                       dim3((unsigned)nblocks), dim3(256), 0, st, f);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "finalize kernel launch failed: %s",
                hipGetErrorString(e));
  return X3_OK;
}

}  // namespace x3i
