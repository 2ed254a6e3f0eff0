// x3conv.hip -- host side of libx3conv.so: argument validation and the C
// ABI declared in include/x3conv.h.  The kernel configuration for a shape is
// chosen in dispatch.hpp; each epilogue's kernels are instantiated in a
// translation unit of their own (epi_*.hip).
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
#include <mutex>

#include "dispatch.hpp"

#define X3_API extern "C" __attribute__((visibility("default")))

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace x3i {

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

}  // namespace x3i

namespace {

using x3i::fail;

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
  if (Cout > x3::kMaxCout)
    return fail(X3_EUNSUPPORTED, "Cout=%d exceeds %d", Cout, x3::kMaxCout);
  if ((uint64_t)Cin * H * W * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of x must be smaller than 2 GiB");
  if ((uint64_t)Cout * Cin * 9 * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "the weight tensor must be smaller than 2 GiB");
  if (!w || !b) return fail(X3_EINVAL, "null weight or bias pointer");
  if (B > 0 && (!x || !out)) return fail(X3_EINVAL, "null x or out pointer");
  s = Shape{B, Cin, H, W, Cout, H - 2, W - 2};
  return X3_OK;
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

}  // namespace

// ============================================================================
// C ABI

namespace {
// The two channel-min entry points, either layout of x (out [B][Ho][Wo] is
// the same in both).
x3_status conv_channel_min(const float* x, const float* w, const float* b,
                           float scale, float* out, int B, int Cin, int H,
                           int W, int Cout, void* stream, int epi, bool nhwc) {
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
  const hipStream_t st = (hipStream_t)stream;
  if (nhwc) return x3i::launch_nhwc(a, epi, st);
  return epi == x3::EPI_MIN_TANH2 ? x3i::launch_min_tanh2(a, st)
                                  : x3i::launch_scale_min(a, st);
}
}  // namespace

X3_API x3_status x3_conv3x3_min_tanh2_f32(const float* x, const float* w,
                                          const float* b, float* out, int B,
                                          int Cin, int H, int W, int Cout,
                                          void* stream) {
  return conv_channel_min(x, w, b, 1.0f, out, B, Cin, H, W, Cout, stream,
                          x3::EPI_MIN_TANH2, false);
}

X3_API x3_status x3_conv3x3_min_tanh2_nhwc_f32(const float* x, const float* w,
                                               const float* b, float* out,
                                               int B, int Cin, int H, int W,
                                               int Cout, void* stream) {
  return conv_channel_min(x, w, b, 1.0f, out, B, Cin, H, W, Cout, stream,
                          x3::EPI_MIN_TANH2, true);
}

namespace {
// Shared by the exact and the tanh-approximation GELU entry points, and
// (mult == nullptr, store_only) by the plain convolution.
x3_status conv_elementwise(const float* x, const float* w, const float* b,
                           const float* mult, float neg_slope, float* out,
                           int B, int Cin, int H, int W, int Cout, void* stream,
                           bool store_only, bool tanh_form, bool nhwc) {
  Shape s;
  x3_status rc = check_common(x, w, b, out, B, Cin, H, W, Cout, s);
  if (rc != X3_OK) return rc;
  if (!store_only && !mult) return fail(X3_EINVAL, "null multiplier pointer");
  // (channels padded to whole channel blocks must stay addressable too)
  if ((uint64_t)x3i::padded_cout(Cout) * (H - 2) * (W - 2) * 4 >= (1ull << 31))
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
  if (nhwc) {
    if (Cout % 4 == 0 && ((uintptr_t)out & 15u) == 0) a.flags |= x3::kOutVec4;
    return x3i::launch_nhwc(a, x3::EPI_MUL_LRELU_GELU, (hipStream_t)stream);
  }
  if (store_only) return x3i::launch_conv_store(a, (hipStream_t)stream);
  return tanh_form ? x3i::launch_mul_lrelu_gelu_tanh(a, (hipStream_t)stream)
                   : x3i::launch_mul_lrelu_gelu(a, (hipStream_t)stream);
}
}  // namespace

X3_API x3_status x3_conv3x3_bias_f32(const float* x, const float* w,
                                     const float* b, float* y, int B, int Cin,
                                     int H, int W, int Cout, void* stream) {
  return conv_elementwise(x, w, b, nullptr, 0.0f, y, B, Cin, H, W, Cout,
                          stream, true, false, false);
}

X3_API x3_status x3_conv3x3_mul_lrelu_gelu_f32(const float* x, const float* w,
                                               const float* b,
                                               const float* mult,
                                               float neg_slope, float* out,
                                               int B, int Cin, int H, int W,
                                               int Cout, void* stream) {
  return conv_elementwise(x, w, b, mult, neg_slope, out, B, Cin, H, W, Cout,
                          stream, false, false, false);
}

X3_API x3_status x3_conv3x3_mul_lrelu_gelu_nhwc_f32(
    const float* x, const float* w, const float* b, const float* mult,
    float neg_slope, float* out, int B, int Cin, int H, int W, int Cout,
    void* stream) {
  return conv_elementwise(x, w, b, mult, neg_slope, out, B, Cin, H, W, Cout,
                          stream, false, false, true);
}

X3_API x3_status x3_conv3x3_mul_lrelu_gelu_tanh_f32(
    const float* x, const float* w, const float* b, const float* mult,
    float neg_slope, float* out, int B, int Cin, int H, int W, int Cout,
    void* stream) {
  return conv_elementwise(x, w, b, mult, neg_slope, out, B, Cin, H, W, Cout,
                          stream, false, true, false);
}

X3_API x3_status x3_conv3x3_scale_min_f32(const float* x, const float* w,
                                          const float* b, float scale,
                                          float* out, int B, int Cin, int H,
                                          int W, int Cout, void* stream) {
  return conv_channel_min(x, w, b, scale, out, B, Cin, H, W, Cout, stream,
                          x3::EPI_SCALE_MIN, false);
}

X3_API x3_status x3_conv3x3_scale_min_nhwc_f32(const float* x, const float* w,
                                               const float* b, float scale,
                                               float* out, int B, int Cin,
                                               int H, int W, int Cout,
                                               void* stream) {
  return conv_channel_min(x, w, b, scale, out, B, Cin, H, W, Cout, stream,
                          x3::EPI_SCALE_MIN, true);
}

namespace {
// Workspace of the GroupNorm entry point: the statistics partials of the
// fused kernels (windows 1..16), or the whole conv output followed (at a
// 256-byte boundary) by one partial per (sample, channel) plane (larger
// windows, NCHW only).
size_t split_y_bytes(const Shape& s) {
  return ((size_t)s.B * s.Cout * s.Ho * s.Wo * sizeof(float) + 255) / 256 * 256;
}
// Partials the finalize merges per (sample, group): one per wavefront tile,
// times the group's channels where the partials are per channel.
int gn_slots(int Ho, int Wo, int Cin, int Cout, int pool_k, bool nhwc) {
  if (pool_k != 4) return x3i::gn_pps_k(Ho, Wo, pool_k, nhwc);
  return nhwc ? x3i::gn_pps_nhwc(Ho, Wo, Cin, Cout) : x3i::gn_pps(Ho, Wo, Cin, Cout);
}
int gn_parts(const Shape& s, int groups, int pool_k, bool nhwc) {
  const int slots = gn_slots(s.Ho, s.Wo, s.Cin, s.Cout, pool_k, nhwc);
  return x3i::gn_partials_per_channel(s.Cout, groups, pool_k) ? slots * (s.Cout / groups)
                                                              : slots;
}
size_t gn_workspace(const Shape& s, int groups, int pool_k, bool nhwc) {
  if (!x3i::gn_fused_window(pool_k, nhwc))
    return split_y_bytes(s) + (size_t)s.B * s.Cout * sizeof(float4);
  return (size_t)s.B * groups * gn_parts(s, groups, pool_k, nhwc) * sizeof(float4);
}

x3_status check_gn(int B, int Cin, int H, int W, int Cout, int groups,
                   int pool_k, bool nhwc, Shape& s) {
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
  if (Cout > x3::kMaxCout)
    return fail(X3_EUNSUPPORTED, "Cout=%d exceeds %d", Cout, x3::kMaxCout);
  const bool fused = x3i::gn_fused_window(pool_k, nhwc);
  if (nhwc && !fused)
    return fail(X3_EUNSUPPORTED, "NHWC: pool_k=%d not compiled in (1..16)", pool_k);
  if ((uint64_t)Cin * H * W * 4 >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of x must be smaller than 2 GiB");
  // (the kernel works in 64-channel blocks: padded channels and groups
  // must stay addressable too; partials are per group of 4 channels or per
  // channel)
  const uint64_t P = (uint64_t)((H - 2 - pool_k) / pool_k + 1) *
                     ((W - 2 - pool_k) / pool_k + 1);
  const uint64_t cpad = (uint64_t)(Cout + 63) / 64 * 64;
  const uint64_t prows =
      x3i::gn_partials_per_channel(Cout, groups, pool_k) ? cpad : cpad / 4;
  const uint64_t slots = fused ? gn_slots(H - 2, W - 2, Cin, Cout, pool_k, nhwc) : 0;
  if (fused &&
      (cpad * P * 4 >= (1ull << 31) || prows * slots * 16 >= (1ull << 31)))
    return fail(X3_EUNSUPPORTED,
                "one sample of out or of the workspace must be < 2 GiB");
  // larger windows take the split path: the conv output is stored whole
  // (and one group of it is indexed with 32 bits)
  if (!fused && (uint64_t)x3i::padded_cout(Cout) * (H - 2) * (W - 2) * 4 >=
                    (1ull << 31))
    return fail(X3_EUNSUPPORTED, "one sample of the conv output must be < 2 GiB");
  s = Shape{B, Cin, H, W, Cout, H - 2, W - 2};
  return X3_OK;
}
}  // namespace

// ----------------------------------------------------------------------------
// Static device scratch of the allocation-free GroupNorm entry point, for
// callers that cannot allocate device memory.  It holds the partial
// statistics that the caller's workspace holds otherwise.  Every GPU the
// library runs on holds its own copy of `scratch`, at its own address, until
// the process ends.  In host code the array's name is only a host-side
// handle: the device address of the current GPU's copy is looked up once per
// device with hipGetSymbolAddress and kept, and only that address is ever
// handed to a kernel.  Calls on one GPU share the array, so calls that
// overlap in time on one GPU (unordered streams) race.  No kernel needs the
// array cleared: every partial slot a call reads is written earlier in the
// same call.
namespace {
constexpr size_t kScratchBytes = X3_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch (nullptr and an error status
// in `rc` on failure).
void* scratch_address(x3_status& rc) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    rc = fail(X3_EHIP, "no usable current device for the static scratch (%s)",
              e != hipSuccess ? hipGetErrorString(e) : "device id out of range");
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    rc = fail(X3_EHIP, "hipGetSymbolAddress(scratch) failed: %s",
              hipGetErrorString(e));
    return nullptr;
  }
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

namespace {
size_t gn_workspace_query(int B, int Cin, int H, int W, int Cout, int groups,
                          int pool_k, bool nhwc) {
  Shape s;
  char saved[sizeof(g_err)];
  __builtin_memcpy(saved, g_err, sizeof(g_err));
  const x3_status rc = check_gn(B, Cin, H, W, Cout, groups, pool_k, nhwc, s);
  __builtin_memcpy(g_err, saved, sizeof(g_err));
  if (rc != X3_OK) return 0;
  return gn_workspace(s, groups, pool_k, nhwc);
}

x3_status gn_entry(const float* x, const float* w, const float* b,
                   const float* gamma, const float* beta, const float* scale,
                   int groups, float eps, int pool_k, float lo, float hi,
                   float* out, void* workspace, size_t workspace_bytes, int B,
                   int Cin, int H, int W, int Cout, void* stream, bool nhwc,
                   bool use_scratch = false) {
  g_err[0] = '\0';
  Shape s;
  x3_status rc = check_gn(B, Cin, H, W, Cout, groups, pool_k, nhwc, s);
  if (rc != X3_OK) return rc;
  if (!w || !b || !gamma || !beta || !scale)
    return fail(X3_EINVAL, "null weight/bias/gamma/beta/scale pointer");
  if (B > 0 && (!x || !out)) return fail(X3_EINVAL, "null x or out pointer");
  if (!(eps > 0.0f) || !std::isfinite(eps))
    return fail(X3_EINVAL, "eps must be positive and finite");
  if (!std::isfinite(lo) || !std::isfinite(hi) || lo > hi)
    return fail(X3_EINVAL, "clamp bounds must be finite with lo <= hi");
  if (B == 0) return X3_OK;
  const size_t need = gn_workspace(s, groups, pool_k, nhwc);
  if (use_scratch) {
    // the allocation-free entry point: the library's static scratch (its
    // address is looked up once every check has passed)
    if (need > kScratchBytes)
      return fail(X3_EWORKSPACE,
                  "this shape needs %zu bytes of workspace; the static scratch "
                  "of the allocation-free entry point holds %zu",
                  need, kScratchBytes);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(X3_EWORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (((uintptr_t)workspace & 15u) != 0)
      return fail(X3_EINVAL, "workspace must be 16-byte aligned");
  }
  const int Ph = (s.Ho - pool_k) / pool_k + 1, Pw = (s.Wo - pool_k) / pool_k + 1;
  const size_t ob = (size_t)B * Cout * Ph * Pw * 4;
  const size_t cb = s.c_bytes();
  if (overlaps(out, ob, x, s.x_bytes()) || overlaps(out, ob, w, s.w_bytes()) ||
      overlaps(out, ob, b, cb) || overlaps(out, ob, gamma, cb) ||
      overlaps(out, ob, beta, cb) || overlaps(out, ob, scale, cb) ||
      overlaps(out, ob, workspace, need) ||
      overlaps(workspace, need, x, s.x_bytes()) ||
      overlaps(workspace, need, w, s.w_bytes()) ||
      overlaps(workspace, need, b, cb) || overlaps(workspace, need, gamma, cb) ||
      overlaps(workspace, need, beta, cb) || overlaps(workspace, need, scale, cb))
    return fail(X3_EINVAL, "out or workspace overlaps another buffer");
  if (use_scratch) {
    workspace = scratch_address(rc);
    if (!workspace) return rc;
    workspace_bytes = kScratchBytes;
  }

  hipStream_t st = (hipStream_t)stream;
  if (!x3i::gn_fused_window(pool_k, nhwc)) {
    // split path (windows above 16): conv output into the workspace, then
    // the standalone GroupNorm -> scale -> pool -> clamp kernels
    rc = x3i::launch_conv_store(base_args(x, w, b, (float*)workspace, s), st);
    if (rc != X3_OK) return rc;
    x3::GnPlaneArgs g{};
    g.y = (const float*)workspace;
    g.gamma = gamma;
    g.scale = scale;
    g.out = out;
    g.part = (float4*)((char*)workspace + split_y_bytes(s));
    g.C = Cout;
    g.H = s.Ho;
    g.W = s.Wo;
    g.k = pool_k;
    g.Ph = Ph;
    g.Pw = Pw;
    return x3i::launch_epi_gn(g, B, groups, beta, eps, lo, hi, st);
  }
  x3::ConvArgs a = base_args(x, w, b, out, s);
  a.v0 = gamma;
  a.v1 = beta;
  a.v2 = scale;
  a.part = (float4*)workspace;
  a.Ph = Ph;
  a.Pw = Pw;
  a.groups = groups;
  a.pk = pool_k;
  if (pool_k != 4)
    rc = nhwc ? x3i::launch_gn_poolk_nhwc(a, st) : x3i::launch_gn_poolk(a, st);
  else
    rc = nhwc ? x3i::launch_nhwc(a,
                                 x3i::gn_partials_per_channel(Cout, groups)
                                     ? x3::EPI_GN_POOL_CH
                                     : x3::EPI_GN_POOL,
                                 st)
              : x3i::launch_gn_pool(a, st);
  if (rc != X3_OK) return rc;

  x3::GnFinArgs f{};
  f.part = (const float4*)workspace;
  f.gamma = gamma;
  f.beta = beta;
  f.scale = scale;
  f.out = out;
  f.groups = groups;
  f.cpg = Cout / groups;
  f.C = Cout;
  f.pps = gn_parts(s, groups, pool_k, nhwc);
  f.plane = Ph * Pw;
  f.eps = eps;
  f.lo = lo;
  f.hi = hi;
  f.count = (double)f.cpg * s.Ho * s.Wo;
  return nhwc ? x3i::launch_gn_finalize_nhwc(f, B, st)
              : x3i::launch_gn_finalize(f, B * groups, st);
}
}  // namespace

X3_API size_t x3_conv3x3_gn_workspace_bytes(int B, int Cin, int H, int W,
                                            int Cout, int groups, int pool_k) {
  return gn_workspace_query(B, Cin, H, W, Cout, groups, pool_k, false);
}

X3_API size_t x3_conv3x3_gn_nhwc_workspace_bytes(int B, int Cin, int H, int W,
                                                 int Cout, int groups,
                                                 int pool_k) {
  return gn_workspace_query(B, Cin, H, W, Cout, groups, pool_k, true);
}

X3_API x3_status x3_conv3x3_gn_scale_pool_clamp_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, void* workspace, size_t workspace_bytes,
    int B, int Cin, int H, int W, int Cout, void* stream) {
  return gn_entry(x, w, b, gamma, beta, scale, groups, eps, pool_k, lo, hi,
                  out, workspace, workspace_bytes, B, Cin, H, W, Cout, stream,
                  false);
}

X3_API x3_status x3_conv3x3_gn_scale_pool_clamp_noalloc_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, int B, int Cin, int H, int W, int Cout,
    void* stream) {
  return gn_entry(x, w, b, gamma, beta, scale, groups, eps, pool_k, lo, hi,
                  out, nullptr, 0, B, Cin, H, W, Cout, stream, false, true);
}

X3_API x3_status x3_conv3x3_gn_scale_pool_clamp_nhwc_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, void* workspace, size_t workspace_bytes,
    int B, int Cin, int H, int W, int Cout, void* stream) {
  return gn_entry(x, w, b, gamma, beta, scale, groups, eps, pool_k, lo, hi,
                  out, workspace, workspace_bytes, B, Cin, H, W, Cout, stream,
                  true);
}

// ============================================================================
// Standalone epilogues over a stored conv output y [B][C][H][W]

namespace {
// Checks shared by the standalone epilogues.  `out_bytes` is the size of
// the output; inputs are y and the per-channel vectors given.
x3_status check_epi(const float* y, const float* out, int B, int C, int H,
                    int W) {
  g_err[0] = '\0';
  if (B < 0 || C < 1 || H < 1 || W < 1)
    return fail(X3_EINVAL, "sizes must be positive (B >= 0): B=%d C=%d H=%d W=%d",
                B, C, H, W);
  if (B > 0 && (!y || !out)) return fail(X3_EINVAL, "null y or out pointer");
  return X3_OK;
}
}  // namespace

X3_API x3_status x3_epi_min_tanh2_f32(const float* y, float* out, int B, int C,
                                      int H, int W, void* stream) {
  x3_status rc = check_epi(y, out, B, C, H, W);
  if (rc != X3_OK || B == 0) return rc;
  const int64_t P = (int64_t)H * W;
  if (overlaps(out, (size_t)B * P * 4, y, (size_t)B * C * P * 4))
    return fail(X3_EINVAL, "out overlaps y");
  x3::ChanArgs c{};
  c.y = y;
  c.out = out;
  c.C = C;
  c.P = P;
  return x3i::launch_epi_chan(c, x3::CHAN_MIN_TANH2, B, (hipStream_t)stream);
}

X3_API x3_status x3_epi_scale_min_f32(const float* y, float scale, float* out,
                                      int B, int C, int H, int W,
                                      void* stream) {
  x3_status rc = check_epi(y, out, B, C, H, W);
  if (rc != X3_OK) return rc;
  if (!std::isfinite(scale)) return fail(X3_EINVAL, "scale must be finite");
  if (B == 0) return X3_OK;
  const int64_t P = (int64_t)H * W;
  if (overlaps(out, (size_t)B * P * 4, y, (size_t)B * C * P * 4))
    return fail(X3_EINVAL, "out overlaps y");
  x3::ChanArgs c{};
  c.y = y;
  c.out = out;
  c.C = C;
  c.P = P;
  c.scale = scale;
  return x3i::launch_epi_chan(c, x3::CHAN_SCALE_MIN, B, (hipStream_t)stream);
}

namespace {
x3_status epi_gelu(const float* y, const float* mult, float neg_slope,
                   float* out, int B, int C, int H, int W, void* stream,
                   bool tanh_form) {
  x3_status rc = check_epi(y, out, B, C, H, W);
  if (rc != X3_OK) return rc;
  if (!mult) return fail(X3_EINVAL, "null multiplier pointer");
  if (!std::isfinite(neg_slope))
    return fail(X3_EINVAL, "neg_slope must be finite");
  if (B == 0) return X3_OK;
  const int64_t P = (int64_t)H * W;
  const size_t nb = (size_t)B * C * P * 4;
  // out may be y itself, but no other overlap
  if ((out != y && overlaps(out, nb, y, nb)) || overlaps(out, nb, mult, (size_t)C * 4))
    return fail(X3_EINVAL, "out partially overlaps y, or overlaps mult");
  x3::EwArgs e{};
  e.y = y;
  e.mult = mult;
  e.out = out;
  e.C = C;
  e.P = P;
  e.slope = neg_slope;
  return x3i::launch_epi_ew(e, tanh_form, (int64_t)B * C, (hipStream_t)stream);
}
}  // namespace

X3_API x3_status x3_epi_mul_lrelu_gelu_f32(const float* y, const float* mult,
                                           float neg_slope, float* out, int B,
                                           int C, int H, int W, void* stream) {
  return epi_gelu(y, mult, neg_slope, out, B, C, H, W, stream, false);
}

X3_API x3_status x3_epi_mul_lrelu_gelu_tanh_f32(const float* y,
                                                const float* mult,
                                                float neg_slope, float* out,
                                                int B, int C, int H, int W,
                                                void* stream) {
  return epi_gelu(y, mult, neg_slope, out, B, C, H, W, stream, true);
}

X3_API size_t x3_epi_gn_workspace_bytes(int B, int C) {
  if (B < 0 || C < 1) return 0;
  return (size_t)B * C * sizeof(float4);
}

X3_API x3_status x3_epi_gn_scale_pool_clamp_f32(
    const float* y, const float* gamma, const float* beta, const float* scale,
    int groups, float eps, int pool_k, float lo, float hi, float* out,
    void* workspace, size_t workspace_bytes, int B, int C, int H, int W,
    void* stream) {
  x3_status rc = check_epi(y, out, B, C, H, W);
  if (rc != X3_OK) return rc;
  if (groups < 1) return fail(X3_EINVAL, "groups must be >= 1");
  if (pool_k < 1) return fail(X3_EINVAL, "pool_k must be >= 1");
  if (C % groups != 0)
    return fail(X3_ESHAPE, "C=%d is not divisible by groups=%d", C, groups);
  if (H < pool_k || W < pool_k)
    return fail(X3_ESHAPE, "input %dx%d is smaller than the pool window", H, W);
  if ((uint64_t)H * W >= (1ull << 31))
    return fail(X3_EUNSUPPORTED, "a plane of y must hold fewer than 2^31 floats");
  if (!gamma || !beta || !scale)
    return fail(X3_EINVAL, "null gamma/beta/scale pointer");
  if (!(eps > 0.0f) || !std::isfinite(eps))
    return fail(X3_EINVAL, "eps must be positive and finite");
  if (!std::isfinite(lo) || !std::isfinite(hi) || lo > hi)
    return fail(X3_EINVAL, "clamp bounds must be finite with lo <= hi");
  if (B == 0) return X3_OK;
  const size_t need = (size_t)B * C * sizeof(float4);
  if (!workspace || workspace_bytes < need)
    return fail(X3_EWORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)workspace & 15u) != 0)
    return fail(X3_EINVAL, "workspace must be 16-byte aligned");
  const int Ph = (H - pool_k) / pool_k + 1, Pw = (W - pool_k) / pool_k + 1;
  const size_t ob = (size_t)B * C * Ph * Pw * 4, cb = (size_t)C * 4;
  const size_t yb = (size_t)B * C * H * W * 4;
  if (overlaps(out, ob, y, yb) || overlaps(out, ob, gamma, cb) ||
      overlaps(out, ob, beta, cb) || overlaps(out, ob, scale, cb) ||
      overlaps(out, ob, workspace, need) || overlaps(workspace, need, y, yb) ||
      overlaps(workspace, need, gamma, cb) || overlaps(workspace, need, beta, cb) ||
      overlaps(workspace, need, scale, cb))
    return fail(X3_EINVAL, "out or workspace overlaps another buffer");
  x3::GnPlaneArgs g{};
  g.y = y;
  g.gamma = gamma;
  g.scale = scale;
  g.out = out;
  g.part = (float4*)workspace;
  g.C = C;
  g.H = H;
  g.W = W;
  g.k = pool_k;
  g.Ph = Ph;
  g.Pw = Pw;
  return x3i::launch_epi_gn(g, B, groups, beta, eps, lo, hi, (hipStream_t)stream);
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

X3_API x3_status x3_probe_mfma_f32(float* out, int n_out, int iters, void* stream) {
  if (!out) return x3i::fail(X3_EINVAL, "out is NULL");
  if (n_out <= 0 || n_out % 256 != 0)
    return x3i::fail(X3_EINVAL, "n_out must be a positive multiple of 256 (got %d)", n_out);
  if (iters < 1 || iters > 65535)
    return x3i::fail(X3_EINVAL, "iters must be in 1..65535 (got %d)", iters);
  return x3i::launch_mfma_probe(out, n_out / 256, iters, (hipStream_t)stream);
}
