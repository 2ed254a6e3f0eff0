/*
 * x3conv.h -- C ABI of the fused 3x3 convolution + epilogue library for
 * AMD Instinct MI355X (gfx950).  Library: libx3conv.so.
 *
 * Every compute entry point runs one valid 3x3 convolution with bias
 * (stride 1, no padding, dilation 1, groups 1) as an implicit GEMM on the
 * fp32 matrix cores, and applies its epilogue while the convolution result
 * is still in registers, so the full convolution output is never written to
 * device memory.
 *
 * Sources, cited by page and passage (the pages have no numbered sections):
 *   [P25] POPCORNBENCH level-2 problem 25 transcript (Kimi-K2.6): Conv2d
 *         16->64 k3, torch.min over channels with keepdim, tanh, tanh.
 *   [P54] POPCORNBENCH level-2 problem 54 transcript: Conv2d 64->64 k3,
 *         per-channel multiplier [C,1,1], LeakyReLU, GELU (exact erf form).
 *   [P32] POPCORNBENCH level-2 problem 32 transcript: Conv2d 64->128 k3,
 *         multiply by 2.0, min over channels with keepdim; its opening
 *         analysis derives the valid output size H-2.
 *   [P85] POPCORNBENCH level-2 problem 85 transcript: Conv2d 8->64 k3,
 *         GroupNorm(16 groups, eps 1e-5, affine), per-channel scale [C,1,1],
 *         MaxPool2d(4) (stride 4, floor mode), clamp(0, 1).
 *
 * Common conventions
 * ------------------
 * - Every tensor pointer is a DEVICE pointer to contiguous fp32 data that
 *   the caller allocated and owns; the library never allocates, frees or
 *   synchronizes.
 *     x    [B][Cin][H][W]        NCHW
 *     w    [Cout][Cin][3][3]
 *     b    [Cout]
 *   The convolution output y has shape [B][Cout][Ho][Wo], Ho = H-2,
 *   Wo = W-2 ([P32], opening analysis of the reference model):
 *     y[n,co,h,w] = b[co] + sum_{ci,kh,kw} x[n,ci,h+kh,w+kw] * w[co,ci,kh,kw]
 * - `stream` is a hipStream_t (0 = the null stream).  Work is enqueued on it
 *   and the call returns at once; device-side faults surface at the caller's
 *   next synchronization.
 * - Arguments are validated before anything is enqueued.  No call aborts or
 *   prints; the return value is an x3_status and x3_last_error() gives a
 *   thread-local detail string for the last failure on the calling thread.
 * - `out` must not overlap any input.  Inputs are never written.
 * - Supported: 1 <= Cout <= 1024; 3 <= H, W; Cin >= 1; each sample of x
 *   smaller than 2 GiB; every other positive shape works (ragged tiles and
 *   channel counts are masked inside the kernels).  Anything else returns
 *   X3_EUNSUPPORTED.
 * - B == 0 is a valid empty call: nothing is enqueued and X3_OK is returned.
 */
#ifndef X3CONV_H
#define X3CONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int x3_status;
enum {
  X3_OK = 0,            /* enqueued (or nothing to do) */
  X3_EINVAL = 1,        /* null pointer, negative size, non-finite scalar */
  X3_ESHAPE = 2,        /* shape cannot produce an output (H or W < 3, ...) */
  X3_EUNSUPPORTED = 3,  /* valid but not compiled in (e.g. Cout > 1024) */
  X3_EWORKSPACE = 4,    /* workspace missing or too small */
  X3_EHIP = 5           /* the HIP runtime reported an error at launch */
};

/* Epilogue (a), [P25]: out[n,0,h,w] = tanh(tanh(min_co y[n,co,h,w])).
 * out: [B][1][Ho][Wo]. */
x3_status x3_conv3x3_min_tanh2_f32(const float* x, const float* w,
                                   const float* b, float* out, int B, int Cin,
                                   int H, int W, int Cout, void* stream);

/* Epilogue (b), [P54]: v = y[n,co,h,w] * mult[co];
 * v = (v >= 0) ? v : neg_slope * v  (LeakyReLU; the page uses 0.01);
 * out[n,co,h,w] = 0.5 * v * (1 + erf(v / sqrt(2)))  (exact GELU).
 * mult: [Cout] (the page's [Cout,1,1] parameter).  out: [B][Cout][Ho][Wo].
 * neg_slope must be finite (else X3_EINVAL).  One sample of out, with Cout
 * rounded up to the kernel's channel block (64, or 128 when Cout > 64 and
 * that rounds no higher), must be smaller than 2 GiB (else
 * X3_EUNSUPPORTED). */
x3_status x3_conv3x3_mul_lrelu_gelu_f32(const float* x, const float* w,
                                        const float* b, const float* mult,
                                        float neg_slope, float* out, int B,
                                        int Cin, int H, int W, int Cout,
                                        void* stream);

/* Epilogue (b) with the tanh approximation of GELU that [P54] drafts before
 * settling on the erf form: out = 0.5 * v * (1 + tanh(sqrt(2/pi) *
 * (v + 0.044715 * v^3))), v as above.  Same arguments, layouts and errors
 * as x3_conv3x3_mul_lrelu_gelu_f32. */
x3_status x3_conv3x3_mul_lrelu_gelu_tanh_f32(const float* x, const float* w,
                                             const float* b, const float* mult,
                                             float neg_slope, float* out,
                                             int B, int Cin, int H, int W,
                                             int Cout, void* stream);

/* The convolution alone (the first step of every epilogue above, [P32]
 * opening analysis): y = conv3x3(x, w) + b, y: [B][Cout][Ho][Wo].  The
 * starting point of the split path (the standalone epilogues below).  Same
 * limits as x3_conv3x3_mul_lrelu_gelu_f32. */
x3_status x3_conv3x3_bias_f32(const float* x, const float* w, const float* b,
                              float* y, int B, int Cin, int H, int W, int Cout,
                              void* stream);

/* Epilogue (c), [P32]: out[n,0,h,w] = min_co (scale * y[n,co,h,w]).
 * The page uses scale = 2.0; any finite scale is accepted (for scale < 0 the
 * minimum of the scaled values is scale times the channel maximum).
 * out: [B][1][Ho][Wo].  scale must be finite (else X3_EINVAL). */
x3_status x3_conv3x3_scale_min_f32(const float* x, const float* w,
                                   const float* b, float scale, float* out,
                                   int B, int Cin, int H, int W, int Cout,
                                   void* stream);

/* Bytes of device workspace x3_conv3x3_gn_scale_pool_clamp_f32 needs for
 * this shape (partial GroupNorm statistics).  Returns 0 when the shape is
 * invalid or unsupported (the compute call then reports why). */
size_t x3_conv3x3_gn_workspace_bytes(int B, int Cin, int H, int W, int Cout,
                                     int groups, int pool_k);

/* Epilogue (d), [P85]: z = GroupNorm(y; groups, eps, gamma, beta)
 * (per sample and group of Cout/groups consecutive channels: mean and
 * biased variance over those channels and all Ho x Wo positions,
 * (y - mean) / sqrt(var + eps) * gamma[c] + beta[c]); then z * scale[c];
 * then MaxPool2d(pool_k, stride pool_k, no padding, floor mode); then
 * clamp to [lo, hi] as min(max(., lo), hi).
 * gamma, beta, scale: [Cout].  out: [B][Cout][Ph][Pw] with
 * Ph = (Ho - pool_k) / pool_k + 1, Pw = (Wo - pool_k) / pool_k + 1.
 * workspace: device memory of at least x3_conv3x3_gn_workspace_bytes(...)
 * bytes, 16-byte aligned, owned by the caller, contents need not be
 * initialized; it is overwritten, and two calls sharing one workspace must
 * be ordered on one stream.  Two kernels are enqueued on `stream`.  With
 * pool_k in 1..16 the conv kernel writes statistics partials (workspace)
 * and the window extrema (out), then a finalize normalizes out in place.
 * A larger pool_k takes the split path: the conv output goes to the
 * workspace (B*Cout*Ho*Wo floats, then B*Cout 16-byte partials at the next
 * 256-byte boundary), then x3_epi_gn_scale_pool_clamp_f32's kernels run on
 * it.  Supported: any groups dividing Cout (Cout <= 1024), any pool_k >= 1;
 * eps > 0 and finite lo <= hi (else X3_EINVAL); Ho, Wo >= pool_k (else
 * X3_ESHAPE). */
x3_status x3_conv3x3_gn_scale_pool_clamp_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, void* workspace, size_t workspace_bytes,
    int B, int Cin, int H, int W, int Cout, void* stream);

/* Size of the static device scratch of
 * x3_conv3x3_gn_scale_pool_clamp_noalloc_f32 (per GPU). */
#define X3_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc:
 * x3_conv3x3_gn_scale_pool_clamp_f32 (NCHW) without the workspace
 * arguments.  Same operation, arguments, layouts and errors otherwise.  The
 * partial statistics go to a static device array of
 * X3_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; a shape whose workspace
 * (x3_conv3x3_gn_workspace_bytes) exceeds it returns X3_EWORKSPACE.  The
 * call allocates and frees nothing.  The scratch of a GPU is the one of the
 * device current on the calling thread, so `stream` must belong to that
 * device.  All calls on one GPU share its scratch: calls that can overlap
 * in time on one GPU (streams not ordered with each other) race and must
 * not be issued. */
x3_status x3_conv3x3_gn_scale_pool_clamp_noalloc_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, int B, int Cin, int H, int W, int Cout,
    void* stream);

/* ------------------------------------------------------------------------
 * Standalone epilogues over a stored conv output y [B][C][H][W] (NCHW,
 * fp32, device memory owned by the caller).  Each is one HBM-bound kernel;
 * together with x3_conv3x3_bias_f32 they are the unfused form of the fused
 * entry points above (the split strategy that all four pages adopt), and
 * they apply to a convolution computed elsewhere.  Sizes: B >= 0, C, H, W
 * >= 1 (else X3_EINVAL); B == 0 enqueues nothing.  out must not overlap an
 * input (the GELU forms allow out == y exactly).
 * ------------------------------------------------------------------------ */

/* [P25]: out[n,0,h,w] = tanh(tanh(min_c y[n,c,h,w])); out [B][1][H][W]. */
x3_status x3_epi_min_tanh2_f32(const float* y, float* out, int B, int C, int H,
                               int W, void* stream);

/* [P32]: out[n,0,h,w] = min_c (scale * y[n,c,h,w]); out [B][1][H][W]; scale
 * finite (else X3_EINVAL). */
x3_status x3_epi_scale_min_f32(const float* y, float scale, float* out, int B,
                               int C, int H, int W, void* stream);

/* [P54]: out = GELU(LeakyReLU(y * mult[c], neg_slope)), GELU in its exact
 * (erf) form, elementwise;
 * mult [C]; out [B][C][H][W], may be y. */
x3_status x3_epi_mul_lrelu_gelu_f32(const float* y, const float* mult,
                                    float neg_slope, float* out, int B, int C,
                                    int H, int W, void* stream);

/* As above with the tanh approximation of GELU. */
x3_status x3_epi_mul_lrelu_gelu_tanh_f32(const float* y, const float* mult,
                                         float neg_slope, float* out, int B,
                                         int C, int H, int W, void* stream);

/* Bytes of device workspace x3_epi_gn_scale_pool_clamp_f32 needs: one
 * 16-byte partial per (sample, channel) plane (0 for invalid sizes). */
size_t x3_epi_gn_workspace_bytes(int B, int C);

/* [P85]: GroupNorm(groups, eps, gamma, beta) -> * scale[c] ->
 * MaxPool2d(pool_k, stride pool_k, floor) -> clamp[lo, hi], as
 * x3_conv3x3_gn_scale_pool_clamp_f32 defines it, on y.  out [B][C][Ph][Pw],
 * Ph = (H - pool_k) / pool_k + 1, Pw likewise.  groups must divide C and
 * H, W >= pool_k (else X3_ESHAPE); eps > 0, finite lo <= hi (else
 * X3_EINVAL).  workspace: at least x3_epi_gn_workspace_bytes(B, C) bytes,
 * 16-byte aligned, caller-owned, overwritten (else X3_EWORKSPACE /
 * X3_EINVAL).  With pool_k == 4, W even, y 8-byte aligned, C / groups <= 64
 * and a group's pooled block (C / groups * Ph * Pw floats) within 48 KB,
 * one kernel per (sample, group) does everything and the workspace is not
 * touched; otherwise two kernels: per-plane statistics + window extrema
 * (parked in out), then the per-group finalize. */
x3_status x3_epi_gn_scale_pool_clamp_f32(const float* y, const float* gamma,
                                         const float* beta, const float* scale,
                                         int groups, float eps, int pool_k,
                                         float lo, float hi, float* out,
                                         void* workspace,
                                         size_t workspace_bytes, int B, int C,
                                         int H, int W, void* stream);

/* ------------------------------------------------------------------------
 * NHWC (channels-last) input: the same four fused operations with
 *     x    [B][H][W][Cin]   (NHWC, contiguous)
 * and the per-channel outputs channels-last too; w stays [Cout][Cin][3][3]
 * and the per-channel vectors [Cout].  Two pages weigh this layout and keep
 * NCHW: l2_p85 considers channels_last for its convolution, l2_p54 for
 * coalesced staging of its direct convolution (channels contiguous per
 * pixel).  It is the layout PyTorch's channels_last tensors hold.  Arguments,
 * limits and errors are those of the NCHW entry points, except that the
 * GroupNorm form supports pool_k 1..16 (no split path), and windows other
 * than 4 need Cin % 4 == 0 and 16-byte aligned x and w (else
 * X3_EUNSUPPORTED).
 * ------------------------------------------------------------------------ */

/* (a) on NHWC x; out [B][Ho][Wo] (the same bytes in either layout). */
x3_status x3_conv3x3_min_tanh2_nhwc_f32(const float* x, const float* w,
                                        const float* b, float* out, int B,
                                        int Cin, int H, int W, int Cout,
                                        void* stream);

/* (b) on NHWC x; out [B][Ho][Wo][Cout]. */
x3_status x3_conv3x3_mul_lrelu_gelu_nhwc_f32(const float* x, const float* w,
                                             const float* b, const float* mult,
                                             float neg_slope, float* out,
                                             int B, int Cin, int H, int W,
                                             int Cout, void* stream);

/* (c) on NHWC x; out [B][Ho][Wo]. */
x3_status x3_conv3x3_scale_min_nhwc_f32(const float* x, const float* w,
                                        const float* b, float scale,
                                        float* out, int B, int Cin, int H,
                                        int W, int Cout, void* stream);

/* Workspace bytes for x3_conv3x3_gn_scale_pool_clamp_nhwc_f32 (0 when the
 * shape is invalid or unsupported). */
size_t x3_conv3x3_gn_nhwc_workspace_bytes(int B, int Cin, int H, int W,
                                          int Cout, int groups, int pool_k);

/* (d) on NHWC x; out [B][Ph][Pw][Cout]; pool_k 1..16. */
x3_status x3_conv3x3_gn_scale_pool_clamp_nhwc_f32(
    const float* x, const float* w, const float* b, const float* gamma,
    const float* beta, const float* scale, int groups, float eps, int pool_k,
    float lo, float hi, float* out, void* workspace, size_t workspace_bytes,
    int B, int Cin, int H, int W, int Cout, void* stream);

/* Static description of a status code (never NULL). */
const char* x3_status_str(x3_status s);
/* Detail of the last failing call on this thread ("" if none). */
const char* x3_last_error(void);
/* Library version string. */
const char* x3_version(void);

/* Measurement aid, not part of the method: the fp32 matrix-core throughput
 * of a pure MFMA loop, the practical ceiling against which the conv
 * kernels' fractions of the published peak can also be read.  Launches
 * n_out / 256 workgroups of 256 threads; every wavefront runs `iters` rounds
 * of 8 independent v_mfma_f32_32x32x2_f32 chains on constant operands (no
 * memory traffic) and every thread writes one float to out[n_out] (device
 * memory, caller-owned), which is exactly 256 * iters.  Matrix FLOP per
 * call: (n_out / 64) * iters * 8 * 4096.  n_out a positive multiple of 256
 * and 1 <= iters <= 65535, else X3_EINVAL; asynchronous on `stream`. */
x3_status x3_probe_mfma_f32(float* out, int n_out, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* X3CONV_H */
