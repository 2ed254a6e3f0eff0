// dispatch.hpp -- host-side launch of the fused kernels: the choice of the
// kernel configuration for a shape, shared by the per-epilogue translation
// units (epi_*.hip) and the C ABI (x3conv.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "conv3x3_igemm.hpp"
#include "epilogue_kernels.hpp"
#include "x3conv.h"

namespace x3i {

// Set the thread's last-error message and return `s` (defined in x3conv.hip).
x3_status fail(x3_status s, const char* fmt, ...);
// Compute units of the current device.
int num_cus();

// Channel-block width of the kernel configurations: MT = 4 (128 channels
// per pass, 2 N-tiles per wave) when that pads Cout no more than MT = 2
// (64 channels per pass, 4 N-tiles per wave) does, otherwise MT = 2.
inline int channel_block_mt(int Cout) {
  const int p64 = (Cout + 63) / 64 * 64, p128 = (Cout + 127) / 128 * 128;
  return (Cout > 64 && p128 == p64) ? 4 : 2;
}
// Cout rounded up to whole channel blocks of the configuration used.
inline int padded_cout(int Cout) {
  const int cb = 32 * channel_block_mt(Cout);
  return (Cout + cb - 1) / cb * cb;
}

// The 16-byte configurations stage input rows and weight rows with 16-byte
// loads: input rows are 16-byte aligned when W % 4 == 0 (x itself comes
// from the caller's allocator, checked for 16-byte alignment), weight rows
// when Cin % 4 == 0.
inline bool rows_aligned16(const x3::ConvArgs& a) {
  return (a.W % 4 == 0) && (a.Cin % 4 == 0) && (((uintptr_t)a.x & 15u) == 0) &&
         (((uintptr_t)a.w & 15u) == 0);
}

// NHWC x takes 16-byte staging when a pixel's channels start 16-byte
// aligned (Cin % 4 == 0, x aligned) and the weight rows do too.
inline bool nhwc_aligned16(const x3::ConvArgs& a) {
  return (a.Cin % 4 == 0) && (((uintptr_t)a.x & 15u) == 0) &&
         (((uintptr_t)a.w & 15u) == 0);
}
// The NHWC 16-byte configurations that stage permuted weight rows keep a
// flag in bit 30 of each weight offset, so the offsets inside a 128-row
// channel block must stay below 1 GiB (Cin < 233,017); larger Cin takes
// the 4-byte configurations.
inline bool nhwc_x4_weights_fit(const x3::ConvArgs& a) {
  return (int64_t)128 * a.Cin * 9 * 4 < (int64_t(1) << 30);
}

// GroupNorm with pooling windows of any size k (other than 4, which has its
// own epilogue): tiles of 16 x 64 outputs trimmed to whole windows, rows to
// a multiple of k, columns to a multiple of k (NHWC) or of lcm(k, 4) (NCHW:
// tile columns then start on 16-byte boundaries for the 16-byte staging,
// and the partial-slot count does not depend on the alignment of x).
constexpr int kGnkTH = 16, kGnkTWC = 64, kGnkWaves = 8, kGnkMaxWindow = 16;
inline int gnk_rows(int k) { return kGnkTH - kGnkTH % k; }
inline int gnk_cols(int k, bool nhwc) {
  const int g = (k % 4 == 0) ? 4 : (k % 2 == 0 ? 2 : 1);
  const int m = nhwc ? k : k * 4 / g;
  return m > kGnkTWC ? 0 : kGnkTWC - kGnkTWC % m;
}
// Windows the fused GroupNorm kernels pool: 4 (own epilogue) and 1..16.
inline bool gn_fused_window(int k, bool nhwc) {
  return k == 4 || (k >= 1 && k <= kGnkMaxWindow && gnk_cols(k, nhwc) > 0);
}
// partial slots per (sample, group or channel) of the window-k kernels
inline int gn_pps_k(int Ho, int Wo, int k, bool nhwc) {
  if (!gn_fused_window(k, nhwc) || k == 4) return 0;
  const int th = gnk_rows(k), tw = gnk_cols(k, nhwc);
  return ((Ho + th - 1) / th) * ((Wo + tw - 1) / tw) * kGnkWaves;
}

template <class G, int EPI>
x3_status run_conv(x3::ConvArgs a, hipStream_t st) {
  if constexpr (x3::gn_generic_k<EPI>()) {
    static_assert(G::TH == kGnkTH && G::TWC == kGnkTWC && G::NWAVE == kGnkWaves,
                  "window-k tiles");
    if (!(a.pk >= 1 && a.pk <= kGnkMaxWindow) || gnk_cols(a.pk, G::NHWC) <= 0)
      return fail(X3_EUNSUPPORTED, "pool window %d not compiled in", a.pk);
    a.thk = gnk_rows(a.pk);
    a.twk = gnk_cols(a.pk, G::NHWC);
  } else {
    a.thk = G::TH;
    a.twk = G::TWC;
  }
  a.n_rt = (a.Ho + a.thk - 1) / a.thk;
  a.n_ct = (a.Wo + a.twk - 1) / a.twk;
  const int64_t ntiles = (int64_t)a.B * a.n_rt * a.n_ct;
  const int64_t nchunk = (a.Cin + G::CC - 1) / G::CC;
  const int64_t ncb = (a.Cout + G::COUT - 1) / G::COUT;
  if (ncb * G::COUT > x3::kMaxCout)
    return fail(X3_EUNSUPPORTED, "Cout=%d exceeds %d", a.Cout, x3::kMaxCout);
  // weight rows of padded channels are addressed past the end of w: those
  // 32-bit byte offsets must not wrap
  if (ncb * G::COUT * a.Cin * 9 * 4 >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "weights padded to whole channel blocks "
                "must stay below 2 GiB");
  // resident weights: one channel block, at most RC K chunks
  if (G::RESW && (ncb != 1 || nchunk > G::RC))
    return fail(X3_EUNSUPPORTED, "resident-weight configuration misapplied");
  // one workgroup per CU resident (two for the 4-wave configurations and
  // the one-wave small tiles)
  const int cus = num_cus() * (G::NWAVE < 8 ? 2 : 1);
  const int64_t grid = ntiles < cus ? ntiles : cus;
  if (ntiles >= (1ll << 31) || (ntiles / grid + 1) * ncb * nchunk >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "problem too large for 32-bit item counters");
  a.ntiles = (int)ntiles;
  a.nchunk = (int)nchunk;
  a.ncb = (int)ncb;
  hipLaunchKernelGGL((x3::conv3x3_igemm_kernel<G, EPI>), dim3((unsigned)grid),
                     dim3(G::NTHR), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "conv kernel launch failed: %s", hipGetErrorString(e));
  return X3_OK;
}

// Kernel configurations.  All use 8 wavefronts (512 threads, one workgroup
// per CU because of the ~120-140 KB double-buffered LDS stage), CC = 8 input
// channels per K chunk, and wave tiles of 128 accumulators (MT x NW = 8
// MFMA blocks).  The tile width follows the output width.

// 64-channel blocks: 2 channel blocks x 4 N-tiles per wave, TH*NCT = 32.
// (NH: NHWC x, 16-byte staging -- X4 must be set too)
template <int EPI, bool X4, bool NH = false>
x3_status dispatch_mt2(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<2, 8, 4, 8, 8, X4, 0, NH>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<2, 8, 8, 4, 8, X4, 0, NH>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 16, 2, 8, X4, 0, NH>, EPI>(a, st);
  return run_conv<x3::Geo<2, 8, 32, 1, 8, X4, 0, NH>, EPI>(a, st);
}

// 128-channel blocks: 4 channel blocks x 2 N-tiles per wave, TH*NCT = 16.
template <int EPI, bool X4, bool NH = false>
x3_status dispatch_mt4(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<4, 8, 2, 8, 8, X4, 0, NH>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<4, 8, 4, 4, 8, X4, 0, NH>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<4, 8, 8, 2, 8, X4, 0, NH>, EPI>(a, st);
  return run_conv<x3::Geo<4, 8, 16, 1, 8, X4, 0, NH>, EPI>(a, st);
}

// The same tiles with the weights of (up to) two K chunks resident in LDS:
// Cin <= 16 and one channel block (Cout <= 64 or 128).  16-byte staging only.
template <int EPI, bool NH = false>
x3_status dispatch_mt2_rw(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<2, 8, 4, 8, 8, true, 2, NH>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<2, 8, 8, 4, 8, true, 2, NH>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 16, 2, 8, true, 2, NH>, EPI>(a, st);
  return run_conv<x3::Geo<2, 8, 32, 1, 8, true, 2, NH>, EPI>(a, st);
}
template <int EPI, bool NH = false>
x3_status dispatch_mt4_rw(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<4, 8, 2, 8, 8, true, 2, NH>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<4, 8, 4, 4, 8, true, 2, NH>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<4, 8, 8, 2, 8, true, 2, NH>, EPI>(a, st);
  return run_conv<x3::Geo<4, 8, 16, 1, 8, true, 2, NH>, EPI>(a, st);
}

// The 16-byte configurations (NCHW, or NHWC with NH), resident weights
// when they fit: all K chunks of the one channel block.  NHWC with staged
// weights takes 64-channel blocks whenever the GroupNorm partial layout
// does not fix the block: their weight rows are staged in the K walk's
// order (conflict-free fragment reads) where 128-channel blocks keep the
// stored order, and two 64-channel passes beat one 128-channel pass (the
// 64 -> 128 channel-min on [64,64,256,256]: 4.14-4.16 against 4.21 ms).
template <int EPI, bool NH>
x3_status dispatch_x4(const x3::ConvArgs& a, hipStream_t st) {
  const int mt = channel_block_mt(a.Cout);
  if (NH && !x3::gn_epilogue<EPI>() && a.Cin > 16)
    return dispatch_mt2<EPI, true, NH>(a, st);
  if (a.Cin <= 16 && a.Cout <= 32 * mt)
    return mt == 4 ? dispatch_mt4_rw<EPI, NH>(a, st) : dispatch_mt2_rw<EPI, NH>(a, st);
  return mt == 4 ? dispatch_mt4<EPI, true, NH>(a, st) : dispatch_mt2<EPI, true, NH>(a, st);
}

// Problems too small to fill the GPU with the tiles above (at most
// kSmallPixels output pixels, e.g. [2,16,32,32] -> 30x30: two 32x32 tiles
// for 256 CUs): tiles of one row of 32 columns with one wavefront each,
// so the work spreads over many CUs and each wavefront's chain of matrix
// instructions is short.
constexpr int64_t kSmallPixels = 32768;
template <int EPI, bool X4>
x3_status dispatch_small(const x3::ConvArgs& a, hipStream_t st) {
  const int mt = channel_block_mt(a.Cout);
  const bool res = X4 && a.Cin <= 16 && a.Cout <= 32 * mt;
  if (mt == 4)
    return res ? run_conv<x3::Geo<4, 8, 1, 1, 1, true, 2>, EPI>(a, st)
               : run_conv<x3::Geo<4, 8, 1, 1, 1, X4, 0>, EPI>(a, st);
  return res ? run_conv<x3::Geo<2, 8, 1, 1, 1, true, 2>, EPI>(a, st)
             : run_conv<x3::Geo<2, 8, 1, 1, 1, X4, 0>, EPI>(a, st);
}

template <int EPI>
x3_status dispatch(const x3::ConvArgs& a, hipStream_t st) {
  if ((int64_t)a.B * a.Ho * a.Wo <= kSmallPixels)
    return rows_aligned16(a) ? dispatch_small<EPI, true>(a, st)
                             : dispatch_small<EPI, false>(a, st);
  if (rows_aligned16(a)) return dispatch_x4<EPI, false>(a, st);
  if (channel_block_mt(a.Cout) == 4) return dispatch_mt4<EPI, false>(a, st);
  return dispatch_mt2<EPI, false>(a, st);
}

// Per-epilogue launchers, one translation unit each.
x3_status launch_min_tanh2(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_mul_lrelu_gelu(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_scale_min(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_mul_lrelu_gelu_tanh(const x3::ConvArgs& a, hipStream_t st);
// Split path: the conv output as is, and the standalone epilogue kernels.
x3_status launch_conv_store(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_epi_chan(x3::ChanArgs c, int mode, int64_t B, hipStream_t st);
x3_status launch_epi_ew(x3::EwArgs e, bool tanh_form, int64_t planes,
                        hipStream_t st);
// (the plane kernel, then the finalize; g.part holds B*C float4)
x3_status launch_epi_gn(const x3::GnPlaneArgs& g, int64_t B, int groups,
                        const float* beta, float eps, float lo, float hi,
                        hipStream_t st);
// GroupNorm path: the conv pass (partials + pooled extrema), then the
// finalize pass over B*groups workgroups.
x3_status launch_gn_pool(const x3::ConvArgs& a, hipStream_t st);
// The same for pooling windows other than 4 (a.pk, 1..16), NCHW or NHWC x.
x3_status launch_gn_poolk(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_gn_poolk_nhwc(const x3::ConvArgs& a, hipStream_t st);
x3_status launch_gn_finalize(const x3::GnFinArgs& f, int nblocks,
                             hipStream_t st);
// NHWC x: the fused conv with epilogue `epi` (EPI_MIN_TANH2,
// EPI_MUL_LRELU_GELU, EPI_SCALE_MIN, EPI_GN_POOL, EPI_GN_POOL_CH), the NHWC
// GroupNorm finalize, and the GroupNorm partial slots of the NHWC tiles.
x3_status launch_nhwc(const x3::ConvArgs& a, int epi, hipStream_t st);
x3_status launch_gn_finalize_nhwc(x3::GnFinArgs f, int B, hipStream_t st);
// The fp32 MFMA-loop probe (probe.hip), `blocks` workgroups of 256 threads.
x3_status launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st);
int gn_pps_nhwc(int Ho, int Wo, int Cin, int Cout);

// GroupNorm partial slots per (sample, group or channel) for this shape: one
// per wavefront tile of the configuration launch_gn_pool picks.
int gn_pps(int Ho, int Wo, int Cin, int Cout);
// Groups of 4 channels take per-group partials (one lane holds a whole
// group); any other group size takes per-channel partials.
inline bool gn_partials_per_channel(int Cout, int groups) {
  return Cout / groups != 4;
}
// The window-k kernels for k >= 3 (LDS window buffer) always take
// per-channel partials.
inline bool gn_partials_per_channel(int Cout, int groups, int pool_k) {
  return gn_partials_per_channel(Cout, groups) || (pool_k != 4 && pool_k >= 3);
}
// float4 partials per (sample, group) that the finalize merges.
inline int gn_parts_per_group(int Ho, int Wo, int Cin, int Cout, int groups) {
  const int slots = gn_pps(Ho, Wo, Cin, Cout);
  return gn_partials_per_channel(Cout, groups) ? slots * (Cout / groups) : slots;
}

}  // namespace x3i
