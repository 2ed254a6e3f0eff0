// x3conv.hip -- host side of libx3conv.so: argument validation, choice of
// the kernel configuration, and the C ABI declared in include/x3conv.h.
//
// Nothing here allocates, frees or synchronizes device memory: every buffer
// belongs to the caller, and every call only enqueues kernels on the
// caller's stream.
#include "x3conv.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "conv3x3_igemm.hpp"

#define X3_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

x3_status fail(x3_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// Compute units of the current device (cached per device id).
int num_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

struct Shape {
  int B, Cin, H, W, Cout, Ho, Wo;
  size_t x_bytes() const { return (size_t)B * Cin * H * W * 4; }
  size_t w_bytes() const { return (size_t)Cout * Cin * 9 * 4; }
  size_t c_bytes() const { return (size_t)Cout * 4; }
};

// Checks shared by every entry point.  Returns X3_OK and fills `s`.
x3_status check_common(const float* x, const float* w, const float* b,
                       const float* out, int B, int Cin, int H, int W,
                       int Cout, Shape& s) {
  g_err[0] = '\0';
  if (B < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1)
    return fail(X3_EINVAL, "sizes must be positive (B >= 0): B=%d Cin=%d H=%d "
                "W=%d Cout=%d", B, Cin, H, W, Cout);
  if (H < 3 || W < 3)
    return fail(X3_ESHAPE, "a valid 3x3 convolution needs H, W >= 3 (got %dx%d)",
                H, W);
  if (Cout != 64 && Cout != 128)
    return fail(X3_EUNSUPPORTED, "Cout=%d is not compiled in (64 or 128)", Cout);
  if ((uint64_t)Cin * H * W * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of x must be smaller than 2 GiB");
  if ((uint64_t)Cout * Cin * 9 * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "the weight tensor must be smaller than 2 GiB");
  if (!w || !b) return fail(X3_EINVAL, "null weight or bias pointer");
  if (B > 0 && (!x || !out)) return fail(X3_EINVAL, "null x or out pointer");
  s = Shape{B, Cin, H, W, Cout, H - 2, W - 2};
  return X3_OK;
}

// ----------------------------------------------------------------------------
// Kernel configurations.  All use 8 wavefronts (512 threads, one workgroup
// per CU because of the ~120-140 KB double-buffered LDS stage), CC = 8 input
// channels per K chunk, and wave tiles of 128 accumulators (MT x NW = 8
// MFMA blocks).  The tile width follows the output width.

template <class G, int EPI>
x3_status run_conv(x3::ConvArgs a, hipStream_t st) {
  a.n_rt = (a.Ho + G::TH - 1) / G::TH;
  a.n_ct = (a.Wo + G::TWC - 1) / G::TWC;
  const int64_t ntiles = (int64_t)a.B * a.n_rt * a.n_ct;
  const int64_t nchunk = (a.Cin + G::CC - 1) / G::CC;
  // one workgroup per CU resident (two for the 4-wave configurations)
  const int cus = num_cus() * (G::NWAVE == 4 ? 2 : 1);
  const int64_t grid = ntiles < cus ? ntiles : cus;
  if (ntiles >= (1ll << 31) || (ntiles / grid + 1) * nchunk >= (1ll << 31))
    return fail(X3_EUNSUPPORTED, "problem too large for 32-bit tile counters");
  a.ntiles = (int)ntiles;
  a.nchunk = (int)nchunk;
  hipLaunchKernelGGL((x3::conv3x3_igemm_kernel<G, EPI>), dim3((unsigned)grid),
                     dim3(G::NTHR), 0, st, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "conv kernel launch failed: %s", hipGetErrorString(e));
  return X3_OK;
}

// Cout = 64: 2 channel blocks x 4 N-tiles per wave, TH*NCT = 32.
template <int EPI, bool X4>
x3_status dispatch64_(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<2, 8, 4, 8, 8, X4>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<2, 8, 8, 4, 8, X4>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<2, 8, 16, 2, 8, X4>, EPI>(a, st);
  return run_conv<x3::Geo<2, 8, 32, 1, 8, X4>, EPI>(a, st);
}

// Cout = 128: 4 channel blocks x 2 N-tiles per wave, TH*NCT = 16.
template <int EPI, bool X4>
x3_status dispatch128_(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Wo > 128) return run_conv<x3::Geo<4, 8, 2, 8, 8, X4>, EPI>(a, st);
  if (a.Wo > 64) return run_conv<x3::Geo<4, 8, 4, 4, 8, X4>, EPI>(a, st);
  if (a.Wo > 32) return run_conv<x3::Geo<4, 8, 8, 2, 8, X4>, EPI>(a, st);
  return run_conv<x3::Geo<4, 8, 16, 1, 8, X4>, EPI>(a, st);
}

// Input rows are 16-byte aligned when W % 4 == 0 (x itself comes from the
// caller's allocator, checked for 16-byte alignment): then the input is
// staged with 16-byte loads.
bool rows_aligned16(const x3::ConvArgs& a) {
  return (a.W % 4 == 0) && (((uintptr_t)a.x & 15u) == 0);
}

template <int EPI>
x3_status dispatch64(const x3::ConvArgs& a, hipStream_t st) {
  return rows_aligned16(a) ? dispatch64_<EPI, true>(a, st)
                           : dispatch64_<EPI, false>(a, st);
}

template <int EPI>
x3_status dispatch(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Cout == 64) return dispatch64<EPI>(a, st);
  return rows_aligned16(a) ? dispatch128_<EPI, true>(a, st)
                           : dispatch128_<EPI, false>(a, st);
}

x3::ConvArgs base_args(const float* x, const float* w, const float* b,
                       float* out, const Shape& s) {
  x3::ConvArgs a{};
  a.x = x;
  a.w = w;
  a.b = b;
  a.out = out;
  a.B = s.B;
  a.Cin = s.Cin;
  a.H = s.H;
  a.W = s.W;
  a.Cout = s.Cout;
  a.Ho = s.Ho;
  a.Wo = s.Wo;
  return a;
}

// GroupNorm path geometry.  With Cin <= 8 (one K chunk) the weight tile is
// resident and two 4-wave workgroups share a CU; otherwise the 8-wave
// tiles of the Cout = 64 table.  Both have 4-row wave tiles (one row of
// pooling windows).
struct GnGeo {
  int th, twc, nwave;
};
GnGeo gn_geo(int Wo, int Cin) {
  if (Cin <= 8) {
    if (Wo > 64) return {4, 128, 4};
    if (Wo > 32) return {8, 64, 4};
    return {16, 32, 4};
  }
  if (Wo > 128) return {4, 256, 8};
  if (Wo > 64) return {8, 128, 8};
  if (Wo > 32) return {16, 64, 8};
  return {32, 32, 8};
}
int gn_pps(int Ho, int Wo, int Cin) {  // partial slots per (sample, group)
  const GnGeo g = gn_geo(Wo, Cin);
  return ((Ho + g.th - 1) / g.th) * ((Wo + g.twc - 1) / g.twc) * g.nwave;
}

template <bool X4>
x3_status dispatch_gn_(const x3::ConvArgs& a, hipStream_t st) {
  if (a.Cin <= 8) {
    if (a.Wo > 64)
      return run_conv<x3::Geo<2, 8, 4, 4, 4, X4, true>, x3::EPI_GN_POOL>(a, st);
    if (a.Wo > 32)
      return run_conv<x3::Geo<2, 8, 8, 2, 4, X4, true>, x3::EPI_GN_POOL>(a, st);
    return run_conv<x3::Geo<2, 8, 16, 1, 4, X4, true>, x3::EPI_GN_POOL>(a, st);
  }
  return dispatch64_<x3::EPI_GN_POOL, X4>(a, st);
}

x3_status dispatch_gn(const x3::ConvArgs& a, hipStream_t st) {
  return rows_aligned16(a) ? dispatch_gn_<true>(a, st)
                           : dispatch_gn_<false>(a, st);
}

}  // namespace

// ============================================================================
// C ABI

X3_API x3_status x3_conv3x3_min_tanh2_f32(const float* x, const float* w,
                                          const float* b, float* out, int B,
                                          int Cin, int H, int W, int Cout,
                                          void* stream) {
  Shape s;
  x3_status rc = check_common(x, w, b, out, B, Cin, H, W, Cout, s);
  if (rc != X3_OK) return rc;
  if (B == 0) return X3_OK;
  const size_t ob = (size_t)B * s.Ho * s.Wo * 4;
  if (overlaps(out, ob, x, s.x_bytes()) || overlaps(out, ob, w, s.w_bytes()) ||
      overlaps(out, ob, b, s.c_bytes()))
    return fail(X3_EINVAL, "out overlaps an input");
  return dispatch<x3::EPI_MIN_TANH2>(base_args(x, w, b, out, s),
                                     (hipStream_t)stream);
}

X3_API x3_status x3_conv3x3_mul_lrelu_gelu_f32(const float* x, const float* w,
                                               const float* b,
                                               const float* mult,
                                               float neg_slope, float* out,
                                               int B, int Cin, int H, int W,
                                               int Cout, void* stream) {
  Shape s;
  x3_status rc = check_common(x, w, b, out, B, Cin, H, W, Cout, s);
  if (rc != X3_OK) return rc;
  if (!mult) return fail(X3_EINVAL, "null multiplier pointer");
  if ((uint64_t)Cout * (H - 2) * (W - 2) * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of out must be smaller than 2 GiB");
  if (!std::isfinite(neg_slope))
    return fail(X3_EINVAL, "neg_slope must be finite");
  if (B == 0) return X3_OK;
  const size_t ob = (size_t)B * Cout * s.Ho * s.Wo * 4;
  if (overlaps(out, ob, x, s.x_bytes()) || overlaps(out, ob, w, s.w_bytes()) ||
      overlaps(out, ob, b, s.c_bytes()) || overlaps(out, ob, mult, s.c_bytes()))
    return fail(X3_EINVAL, "out overlaps an input");
  x3::ConvArgs a = base_args(x, w, b, out, s);
  a.v0 = mult;
  a.s0 = neg_slope;
  return dispatch<x3::EPI_MUL_LRELU_GELU>(a, (hipStream_t)stream);
}

X3_API x3_status x3_conv3x3_scale_min_f32(const float* x, const float* w,
                                          const float* b, float scale,
                                          float* out, int B, int Cin, int H,
                                          int W, int Cout, void* stream) {
  Shape s;
  x3_status rc = check_common(x, w, b, out, B, Cin, H, W, Cout, s);
  if (rc != X3_OK) return rc;
  if (!std::isfinite(scale)) return fail(X3_EINVAL, "scale must be finite");
  if (B == 0) return X3_OK;
  const size_t ob = (size_t)B * s.Ho * s.Wo * 4;
  if (overlaps(out, ob, x, s.x_bytes()) || overlaps(out, ob, w, s.w_bytes()) ||
      overlaps(out, ob, b, s.c_bytes()))
    return fail(X3_EINVAL, "out overlaps an input");
  x3::ConvArgs a = base_args(x, w, b, out, s);
  a.s0 = scale;
  return dispatch<x3::EPI_SCALE_MIN>(a, (hipStream_t)stream);
}

namespace {
x3_status check_gn(int B, int Cin, int H, int W, int Cout, int groups,
                   int pool_k, Shape& s) {
  if (B < 0 || Cin < 1 || H < 1 || W < 1 || Cout < 1)
    return fail(X3_EINVAL, "sizes must be positive (B >= 0)");
  if (groups < 1) return fail(X3_EINVAL, "groups must be >= 1");
  if (pool_k < 1) return fail(X3_EINVAL, "pool_k must be >= 1");
  if (H < 3 || W < 3) return fail(X3_ESHAPE, "H, W must be >= 3");
  if (Cout % groups != 0)
    return fail(X3_ESHAPE, "Cout=%d is not divisible by groups=%d", Cout,
                groups);
  if (H - 2 < pool_k || W - 2 < pool_k)
    return fail(X3_ESHAPE, "conv output %dx%d is smaller than the pool window",
                H - 2, W - 2);
  if (Cout != 64)
    return fail(X3_EUNSUPPORTED, "GroupNorm path: Cout=%d not compiled in (64)",
                Cout);
  if (Cout / groups != 4)
    return fail(X3_EUNSUPPORTED,
                "GroupNorm path: %d channels per group not compiled in (4)",
                Cout / groups);
  if (pool_k != 4)
    return fail(X3_EUNSUPPORTED, "pool_k=%d not compiled in (4)", pool_k);
  if ((uint64_t)Cin * H * W * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of x must be smaller than 2 GiB");
  const uint64_t P = (uint64_t)((H - 2 - pool_k) / pool_k + 1) *
                     ((W - 2 - pool_k) / pool_k + 1);
  if ((uint64_t)Cout * P * 4 >= (1ull << 31) ||
      (uint64_t)groups * gn_pps(H - 2, W - 2, Cin) * 16 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED,
                "one sample of out or of the workspace must be < 2 GiB");
  s = Shape{B, Cin, H, W, Cout, H - 2, W - 2};
  return X3_OK;
}
}  // namespace

X3_API size_t x3_conv3x3_gn_workspace_bytes(int B, int Cin, int H, int W,
                                            int Cout, int groups, int pool_k) {
  Shape s;
  char saved[sizeof(g_err)];
  __builtin_memcpy(saved, g_err, sizeof(g_err));
  const x3_status rc = check_gn(B, Cin, H, W, Cout, groups, pool_k, s);
  __builtin_memcpy(g_err, saved, sizeof(g_err));
  if (rc != X3_OK) return 0;
  return (size_t)B * groups * gn_pps(s.Ho, s.Wo, s.Cin) * sizeof(float4);
}

X3_API x3_status x3_conv3x3_gn_scale_pool_clamp_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, void* workspace, size_t workspace_bytes,
    int B, int Cin, int H, int W, int Cout, void* stream) {
  g_err[0] = '\0';
  Shape s;
  x3_status rc = check_gn(B, Cin, H, W, Cout, groups, pool_k, s);
  if (rc != X3_OK) return rc;
  if (!w || !b || !gamma || !beta || !scale)
    return fail(X3_EINVAL, "null weight/bias/gamma/beta/scale pointer");
  if (B > 0 && (!x || !out)) return fail(X3_EINVAL, "null x or out pointer");
  if (!(eps > 0.0f) || !std::isfinite(eps))
    return fail(X3_EINVAL, "eps must be positive and finite");
  if (!std::isfinite(lo) || !std::isfinite(hi) || lo > hi)
    return fail(X3_EINVAL, "clamp bounds must be finite with lo <= hi");
  if (B == 0) return X3_OK;
  const size_t need = (size_t)B * groups * gn_pps(s.Ho, s.Wo, s.Cin) * sizeof(float4);
  if (!workspace || workspace_bytes < need)
    return fail(X3_EWORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 15u) != 0)
    return fail(X3_EINVAL, "workspace must be 16-byte aligned");
  const int Ph = (s.Ho - pool_k) / pool_k + 1, Pw = (s.Wo - pool_k) / pool_k + 1;
  const size_t ob = (size_t)B * Cout * Ph * Pw * 4;
  const size_t cb = s.c_bytes();
  if (overlaps(out, ob, x, s.x_bytes()) || overlaps(out, ob, w, s.w_bytes()) ||
      overlaps(out, ob, b, cb) || overlaps(out, ob, gamma, cb) ||
      overlaps(out, ob, beta, cb) || overlaps(out, ob, scale, cb) ||
      overlaps(out, ob, workspace, need) ||
      overlaps(workspace, need, x, s.x_bytes()) ||
      overlaps(workspace, need, w, s.w_bytes()))
    return fail(X3_EINVAL, "out or workspace overlaps another buffer");

  hipStream_t st = (hipStream_t)stream;
  x3::ConvArgs a = base_args(x, w, b, out, s);
  a.v0 = gamma;
  a.v1 = beta;
  a.v2 = scale;
  a.part = (float4*)workspace;
  a.Ph = Ph;
  a.Pw = Pw;
  a.groups = groups;
  rc = dispatch_gn(a, st);
  if (rc != X3_OK) return rc;

  x3::GnFinArgs f{};
  f.part = (const float4*)workspace;
  f.gamma = gamma;
  f.beta = beta;
  f.scale = scale;
  f.out = out;
  f.groups = groups;
  f.cpg = Cout / groups;
  f.pps = gn_pps(s.Ho, s.Wo, s.Cin);
  f.plane = Ph * Pw;
  f.eps = eps;
  f.lo = lo;
  f.hi = hi;
  f.count = (double)f.cpg * s.Ho * s.Wo;
  // The finalize moves each group's pooled block as float4 when it is
  // 16-byte aligned (4 channels per group make every block a multiple of 4
  // floats; `out` itself must be aligned).
  if (((uintptr_t)out & 15u) == 0 && (f.cpg * f.plane) % 4 == 0)
    hipLaunchKernelGGL((x3::gn_finalize_kernel<256, true>),
                       dim3((unsigned)(B * groups)), dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL((x3::gn_finalize_kernel<256, false>),
                       dim3((unsigned)(B * groups)), dim3(256), 0, st, f);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(X3_EHIP, "finalize kernel launch failed: %s",
                hipGetErrorString(e));
  return X3_OK;
}

X3_API const char* x3_status_str(x3_status s) {
  switch (s) {
    case X3_OK: return "ok";
    case X3_EINVAL: return "invalid argument";
    case X3_ESHAPE: return "invalid shape";
    case X3_EUNSUPPORTED: return "unsupported configuration";
    case X3_EWORKSPACE: return "workspace missing or too small";
    case X3_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

X3_API const char* x3_last_error(void) { return g_err; }

X3_API const char* x3_version(void) { return "x3conv 0.1.0 (gfx950)"; }
