// epi_split.hip -- the split path: the conv kernel storing its output (with
// bias) as is, and the launches of the standalone epilogue kernels.
#include "dispatch.hpp"
#include "epilogue_kernels.hpp"

namespace x3i {
namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

x3_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return X3_OK;
}

}  // namespace

x3_status launch_conv_store(const x3::ConvArgs& a, hipStream_t st) {
  return dispatch<x3::EPI_STORE>(a, st);
}

x3_status launch_epi_chan(x3::ChanArgs c, int mode, int64_t B, hipStream_t st) {
  const bool vec = c.P % 4 == 0 && aligned16(c.y) && aligned16(c.out);
  const int64_t per = vec ? c.P / 4 : c.P;
  c.nchunk = (per + x3::kEpiThreads - 1) / x3::kEpiThreads;
  const int64_t blocks = B * c.nchunk;
  if (blocks >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "too many pixels for one launch");
  const dim3 grid((unsigned)blocks), block(x3::kEpiThreads);
  if (mode == x3::CHAN_MIN_TANH2) {
    if (vec)
      hipLaunchKernelGGL((x3::chan_extremum_kernel<x3::CHAN_MIN_TANH2, true>), grid, block, 0, st, c);
    else
      hipLaunchKernelGGL((x3::chan_extremum_kernel<x3::CHAN_MIN_TANH2, false>), grid, block, 0, st, c);
  } else {
    if (vec)
      hipLaunchKernelGGL((x3::chan_extremum_kernel<x3::CHAN_SCALE_MIN, true>), grid, block, 0, st, c);
    else
      hipLaunchKernelGGL((x3::chan_extremum_kernel<x3::CHAN_SCALE_MIN, false>), grid, block, 0, st, c);
  }
  return launched("channel-extremum kernel");
}

x3_status launch_epi_ew(x3::EwArgs e, bool tanh_form, int64_t planes,
                        hipStream_t st) {
  const bool vec = e.P % 4 == 0 && aligned16(e.y) && aligned16(e.out);
  const int64_t per = vec ? e.P / 4 : e.P;
  const int64_t span = (int64_t)x3::kEpiThreads * x3::kEwPerThread;
  if (vec && per >= span) {
    // flat form: whole 16 KB blocks over the tensor (see the kernel)
    e.total4 = per * planes;
    const int64_t nblk = (e.total4 + span - 1) / span;
    if (nblk >= (1ll << 31))
      return fail(X3_EUNSUPPORTED, "too many elements for one launch");
    if (tanh_form)
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_flat4_kernel<true>), dim3((unsigned)nblk),
                         dim3(x3::kEpiThreads), 0, st, e);
    else
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_flat4_kernel<false>), dim3((unsigned)nblk),
                         dim3(x3::kEpiThreads), 0, st, e);
    return launched("elementwise epilogue kernel");
  }
  e.nchunk = (per + span - 1) / span;
  const int64_t blocks = planes * e.nchunk;
  if (blocks >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "too many elements for one launch");
  const dim3 grid((unsigned)blocks), block(x3::kEpiThreads);
  if (tanh_form) {
    if (vec)
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_kernel<true, true>), grid, block, 0, st, e);
    else
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_kernel<true, false>), grid, block, 0, st, e);
  } else {
    if (vec)
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_kernel<false, true>), grid, block, 0, st, e);
    else
      hipLaunchKernelGGL((x3::mul_lrelu_gelu_kernel<false, false>), grid, block, 0, st, e);
  }
  return launched("elementwise epilogue kernel");
}

x3_status launch_epi_gn(const x3::GnPlaneArgs& g, int64_t B, int groups,
                        const float* beta, float eps, float lo, float hi,
                        hipStream_t st) {
  const int64_t planes = B * g.C;
  if (planes >= (1ll << 31) || B * groups >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "too many planes for one launch");
  const dim3 grid((unsigned)planes), block(x3::kEpiThreads);
  const int cpg = g.C / groups;
  const int64_t ext_bytes = (int64_t)cpg * g.Ph * g.Pw * 4;
  if (g.k == 4 && g.W % 2 == 0 && ((uintptr_t)g.y & 7u) == 0 &&
      cpg <= x3::kGnGroupMaxCpg && ext_bytes <= x3::kGnGroupMaxLdsBytes) {
    // one kernel: statistics, extrema and normalization per (sample, group)
    x3::GnGroupArgs q{};
    q.y = g.y;
    q.gamma = g.gamma;
    q.beta = beta;
    q.scale = g.scale;
    q.out = g.out;
    q.C = g.C;
    q.H = g.H;
    q.W = g.W;
    q.Ph = g.Ph;
    q.Pw = g.Pw;
    q.cpg = cpg;
    q.eps = eps;
    q.lo = lo;
    q.hi = hi;
    hipLaunchKernelGGL((x3::gn_group_k4w2_kernel<4>), dim3((unsigned)(B * groups)), block,
                       (unsigned)ext_bytes, st, q);
    return launched("GroupNorm group kernel");
  }
  if (g.k == 4 && g.W % 2 == 0 && ((uintptr_t)g.y & 7u) == 0)
    hipLaunchKernelGGL((x3::gn_plane_k4w2_kernel<4>), grid, block, 0, st, g);
  else if (g.k == 4)
    hipLaunchKernelGGL((x3::gn_plane_kernel<4>), grid, block, 0, st, g);
  else
    hipLaunchKernelGGL((x3::gn_plane_kernel<0>), grid, block, 0, st, g);
  const x3_status rc = launched("GroupNorm plane kernel");
  if (rc != X3_OK) return rc;
  // the finalize of the fused path: merge each group's cpg plane partials,
  // then normalize, scale and clamp the parked extrema in place
  x3::GnFinArgs f{};
  f.part = g.part;
  f.gamma = g.gamma;
  f.beta = beta;
  f.scale = g.scale;
  f.out = g.out;
  f.groups = groups;
  f.cpg = g.C / groups;
  f.pps = f.cpg;
  f.plane = g.Ph * g.Pw;
  f.eps = eps;
  f.lo = lo;
  f.hi = hi;
  f.count = (double)f.cpg * g.H * g.W;
  return launch_gn_finalize(f, (int)(B * groups), st);
}

}  // namespace x3i
