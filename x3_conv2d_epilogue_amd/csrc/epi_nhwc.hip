// epi_nhwc.hip -- the fused kernels for NHWC (channels-last) x, and the
// NHWC GroupNorm finalize.  With Cin % 4 == 0 (and 16-byte aligned x and
// w) the input tile is staged with 16-byte direct-to-LDS loads in two
// channel-half regions (4 channels per pixel each) and the kernels take
// the tiles of the NCHW ones; otherwise it is staged pixel-major with a
// 10-dword pixel pitch (8 channels + 2 padding) and 4-byte loads, in tiles
// of at most 128 columns (the pixel-major tile is 1.25x the size of the
// channel-major one).  The MFMA loop and the epilogues are those of the
// NCHW kernels.
#include "dispatch.hpp"

namespace x3i {
namespace {

template <int MT, int TH, int NCT>
using GeoN = x3::Geo<MT, 8, TH, NCT, 8, false, 0, true>;
// GroupNorm with Cin <= 8 and Cout <= 64: resident weights, two 4-wave
// workgroups per CU, tiles of at most 64 columns (LDS: 78 KB each)
template <int TH, int NCT>
using GeoNR = x3::Geo<2, 8, TH, NCT, 4, false, 1, true>;

bool gn_resident_nhwc(int Cin, int Cout) { return Cin <= 8 && Cout <= 64; }

template <int EPI>
x3_status dispatch_nhwc_mt2(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 64) return run_conv<GeoN<2, 8, 4>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<GeoN<2, 16, 2>, EPI>(a, st);
  return run_conv<GeoN<2, 32, 1>, EPI>(a, st);
}

template <int EPI>
x3_status dispatch_nhwc(const x3::ConvArgs& a, hipStream_t st) {
  if (nhwc_aligned16(a) && nhwc_x4_weights_fit(a)) return dispatch_x4<EPI, true>(a, st);
  if (channel_block_mt(a.Cout) == 4) {
    if (a.Wo > 64) return run_conv<GeoN<4, 4, 4>, EPI>(a, st);
    if (a.Wo > 32) return run_conv<GeoN<4, 8, 2>, EPI>(a, st);
    return run_conv<GeoN<4, 16, 1>, EPI>(a, st);
  }
  return dispatch_nhwc_mt2<EPI>(a, st);
}

// (the 16-byte configurations take the same tile shapes as the 4-byte
// ones, so the GroupNorm partial slots do not depend on the alignment)
template <int EPI>
x3_status dispatch_gn_nhwc(const x3::ConvArgs& a, hipStream_t st) {
  if (nhwc_aligned16(a) && nhwc_x4_weights_fit(a)) {
    if (gn_resident_nhwc(a.Cin, a.Cout)) {
      if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 8, 2, 4, true, 1, true>, EPI>(a, st);
      return run_conv<x3::Geo<2, 8, 16, 1, 4, true, 1, true>, EPI>(a, st);
    }
    if (a.Wo > 64) return run_conv<x3::Geo<2, 8, 8, 4, 8, true, 0, true>, EPI>(a, st);
    if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 0, true>, EPI>(a, st);
    return run_conv<x3::Geo<2, 8, 32, 1, 8, true, 0, true>, EPI>(a, st);
  }
  if (gn_resident_nhwc(a.Cin, a.Cout)) {
    if (a.Wo > 32) return run_conv<GeoNR<8, 2>, EPI>(a, st);
    return run_conv<GeoNR<16, 1>, EPI>(a, st);
  }
  return dispatch_nhwc_mt2<EPI>(a, st);
}

}  // namespace

int gn_pps_nhwc(int Ho, int Wo, int Cin, int Cout) {
  if (gn_resident_nhwc(Cin, Cout)) {
    const int th = Wo > 32 ? 8 : 16, twc = Wo > 32 ? 64 : 32;
    return ((Ho + th - 1) / th) * ((Wo + twc - 1) / twc) * 4;
  }
  const int th = Wo > 64 ? 8 : (Wo > 32 ? 16 : 32);
  const int twc = Wo > 64 ? 128 : (Wo > 32 ? 64 : 32);
  return ((Ho + th - 1) / th) * ((Wo + twc - 1) / twc) * 8;
}

x3_status launch_nhwc(const x3::ConvArgs& a, int epi, hipStream_t st) {
  switch (epi) {
    case x3::EPI_MIN_TANH2: return dispatch_nhwc<x3::EPI_MIN_TANH2>(a, st);
    case x3::EPI_MUL_LRELU_GELU: return dispatch_nhwc<x3::EPI_MUL_LRELU_GELU>(a, st);
    case x3::EPI_SCALE_MIN: return dispatch_nhwc<x3::EPI_SCALE_MIN>(a, st);
    case x3::EPI_GN_POOL: return dispatch_gn_nhwc<x3::EPI_GN_POOL>(a, st);
    case x3::EPI_GN_POOL_CH: return dispatch_gn_nhwc<x3::EPI_GN_POOL_CH>(a, st);
    default: return fail(X3_EUNSUPPORTED, "epilogue %d has no NHWC form", epi);
  }
}

x3_status launch_gn_finalize_nhwc(x3::GnFinArgs f, int B, hipStream_t st) {
  const bool vec = f.C % 4 == 0 && ((uintptr_t)f.out & 15u) == 0;
  const int64_t per = (int64_t)f.plane * f.C / (vec ? 4 : 1);
  const int64_t span = (int64_t)x3::kFinNhwcThreads * x3::kFinNhwcPerThread;
  f.nchunk = (int)((per + span - 1) / span);
  const int64_t blocks = (int64_t)B * f.nchunk;
  if (blocks >= (1ll << 31) || (int64_t)f.plane * f.C >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "pooled output too large for one launch");
  if (vec)
    hipLaunchKernelGGL((x3::gn_finalize_nhwc_kernel<x3::kFinNhwcThreads, true>),
                       dim3((unsigned)blocks), dim3(x3::kFinNhwcThreads), 0, st, f);
  else
    hipLaunchKernelGGL((x3::gn_finalize_nhwc_kernel<x3::kFinNhwcThreads, false>),
                       dim3((unsigned)blocks), dim3(x3::kFinNhwcThreads), 0, st, f);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "finalize kernel launch failed: %s",
                hipGetErrorString(e));
  return X3_OK;
}

}  // namespace x3i
