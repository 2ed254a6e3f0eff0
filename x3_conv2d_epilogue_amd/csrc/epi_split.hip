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

x3_status launch_epi_gn(const x3::GnPoolArgs& g, int64_t blocks, hipStream_t st) {
  if (blocks >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "too many (sample, group) pairs for one launch");
  const int64_t total = (int64_t)g.cpg * g.H * g.W;
  const dim3 grid((unsigned)blocks), block(x3::kEpiThreads);
  if (total % 4 == 0 && aligned16(g.y))
    hipLaunchKernelGGL((x3::gn_pool_kernel<true>), grid, block, 0, st, g);
  else
    hipLaunchKernelGGL((x3::gn_pool_kernel<false>), grid, block, 0, st, g);
  return launched("GroupNorm pooling kernel");
}

}  // namespace x3i
